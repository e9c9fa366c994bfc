"""The parity checker (oracle/compare.py) against hand-worked cases, and
plausible mistakes planted in copies of it that some pin must catch."""
import importlib.util
import os
import tempfile

import pytest

import oracle
from oracle import compare
from compare_pins import ALL_PINS

SOURCE = os.path.join(os.path.dirname(oracle.__file__), "compare.py")


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(compare)


# (name, anchor text in compare.py, replacement)
MUTANTS = [
    ("parting_level_plus_one", "return D - diff.bit_length()", "return D - diff.bit_length() + 1"),
    ("parting_level_minus_one", "return D - diff.bit_length()", "return D - diff.bit_length() - 1"),
    ("parting_level_lowest_bit", "return D - diff.bit_length()", "return D - (diff & -diff).bit_length()"),
    ("tie_band_open", "(excused if abs(a) <= thr else bad)", "(excused if abs(a) < thr else bad)"),
    ("tie_band_signed", "(excused if abs(a) <= thr else bad)", "(excused if a <= thr else bad)"),
    ("out_of_range_leaf_allowed", "        if leaf < 0 or leaf >= (1 << D):\n            bad.append",
     "        if leaf < 0:\n            bad.append"),
    ("excused_tokens_kept_in_y", "for t, _, _ in excused + bad:", "for t, _, _ in bad:"),
    ("floor_dropped", "den = np.maximum(np.abs(y_ref), rms)", "den = np.abs(y_ref)"),
    ("magnitude_dropped", "den = np.maximum(np.abs(y_ref), rms)", "den = np.maximum(y_ref, rms)"),
    ("rms_per_column", "rms = np.sqrt(np.mean(y_ref * y_ref, axis=1, keepdims=True))",
     "rms = np.sqrt(np.mean(y_ref * y_ref, axis=0, keepdims=True))"),
    ("rows_ok_ignored", "if rows_ok is not None:", "if False:"),
    ("zero_row_not_absolute", "den = np.where(den > 0, den, 1.0)", "den = np.where(den > 0, den, np.inf)"),
    ("normwise_unscaled", "np.linalg.norm(y_dev - y_ref, axis=1) / nrm", "np.linalg.norm(y_dev - y_ref, axis=1)"),
    ("signs_tie_excuse_dropped", "if took_right != want_right and not abs(a) <= thr:",
     "if took_right != want_right:"),
    ("signs_direction_reversed", "want_right = 0 if a < 0 else 1", "want_right = 1 if a < 0 else 0"),
    ("signs_bits_reversed", "took_right = (leaf >> (D - 1 - lvl)) & 1", "took_right = (leaf >> lvl) & 1"),
    ("signs_pruned_preference_ignored", "want_right ^= 1  # a pruned", "want_right ^= 0  # a pruned"),
    ("signs_dead_child_allowed", "if not node_alive[p, 2 * n + 1 + took_right]:",
     "if False and not node_alive[p, 2 * n + 1 + took_right]:"),
    ("alive_is_and", "alive[:, n] = alive[:, 2 * n + 1] | alive[:, 2 * n + 2]",
     "alive[:, n] = alive[:, 2 * n + 1] & alive[:, 2 * n + 2]"),
    ("signs_out_of_range_allowed", "        if leaf < 0 or leaf >= (1 << D):\n                viol.append",
     "        if leaf < 0:\n                viol.append"),
]


def _load_mutant(path):
    spec = importlib.util.spec_from_file_location("compare_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,anchor,replacement", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, anchor, replacement):
    with open(SOURCE) as f:
        src = f.read()
    assert src.count(anchor) == 1, f"anchor for {name} must occur exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, f"compare_{name}.py")
        with open(path, "w") as f:
            f.write(src.replace(anchor, replacement))
        mod = _load_mutant(path)
        caught = []
        for pin in ALL_PINS:
            try:
                pin(mod)
            except Exception:
                caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
