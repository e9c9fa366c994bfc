"""Pins for ``oracle/compare.py``, the checker that decides what counts as a
parity pass.  Each ``pin_*`` takes the module under test (the real one, or a
mutant copy built by tests/test_compare_mutants.py) and raises
AssertionError when it disagrees with a value worked out by hand here.

What is fixed independently of the checker's code:
* the sign rule (explainer page, gist.science, section 2): right iff the
  logit is not below zero, so a logit of exactly 0 goes right;
* the leaf encoding of the library's interface: bit (D-1-l) is the level-l
  decision, so two leaves first part at the level of their highest
  differing bit;
* the near-tie band |a| <= 1e-4 ||x|| ||w|| (closed at the threshold);
* the RMS-floored relative error, evaluated by hand on two-element rows.
"""
from __future__ import annotations

import math

import numpy as np


def _close(got, want, tol=1e-12):
    assert abs(got - want) <= tol * max(1.0, abs(want)), (got, want)


def pin_parting_level(cmp):
    # D = 3: leaves 0b101 and 0b001 differ in bit 2 -> level 0; 0b100 and
    # 0b101 in bit 0 -> level 2 = D-1; 0b111 and 0b101 in bit 1 -> level 1.
    assert cmp.parting_level(0b101, 0b001, 3) == 0
    assert cmp.parting_level(0b100, 0b101, 3) == 2
    assert cmp.parting_level(0b111, 0b101, 3) == 1
    assert cmp.parting_level(0, 63, 6) == 0
    assert cmp.parting_level(62, 63, 6) == 5
    assert cmp.parting_level(0b010110, 0b011110, 6) == 2


def _ref_d3():
    """A hand-made reference for D = 3, 5 tokens, 2 trees: every oracle
    leaf 0b101, threshold 1 everywhere, logits far from ties (5) except
    where a case puts one."""
    T, P, D = 5, 2, 3
    ref = {"path": np.full((T, P), 0b101, dtype=np.int32),
           "rec_a": np.full((T, P, D + 1), 5.0),
           "rec_thr": np.ones((T, P, D + 1))}
    dev = ref["path"].copy()
    # token 0, tree 0: parts at level 0 with |a| = 0.999 <= 1 -> excused.
    dev[0, 0] = 0b001
    ref["rec_a"][0, 0, 0] = 0.999
    # token 1, tree 1: parts at level 2 (= D-1) with a = -1 exactly at the
    # threshold -> excused (the band is closed).
    dev[1, 1] = 0b100
    ref["rec_a"][1, 1, 2] = -1.0
    # token 2, tree 0: parts at level 1 with |a| = 1.001 -> a failure; its
    # neighbouring levels hold near-ties, so reading the wrong level would
    # excuse it.
    dev[2, 0] = 0b111
    ref["rec_a"][2, 0, 1] = 1.001
    ref["rec_a"][2, 0, 0] = 0.5
    ref["rec_a"][2, 0, 2] = -0.5
    # token 3, tree 1: a leaf index outside [0, 8) -> a failure.
    dev[3, 1] = 8
    # token 3, tree 0: parts at level 2 on a = -5, far below the band -> a
    # failure (the band is two-sided: |a|, not a).
    dev[3, 0] = 0b100
    ref["rec_a"][3, 0, 2] = -5.0
    # token 4 matches everywhere.
    return ref, dev, D


def pin_classify_cases(cmp):
    ref, dev, D = _ref_d3()
    c = cmp.classify_paths(dev, ref, D)
    assert c["mismatches"] == 5
    assert sorted(c["excused"]) == [(0, 0, 0), (1, 1, 2)], c["excused"]
    assert sorted(c["bad"], key=str) == sorted([(2, 0, 1), (3, 0, 2), (3, 1, None)], key=str), c["bad"]
    assert c["flips_near_tie"] == 2
    assert c["tokens_ok"].tolist() == [False, False, False, False, True]


def pin_classify_negative_leaf(cmp):
    ref, dev, D = _ref_d3()
    dev = ref["path"].copy()
    dev[4, 1] = -1
    c = cmp.classify_paths(dev, ref, D)
    assert c["bad"] == [(4, 1, None)] and not c["excused"]
    assert c["tokens_ok"].tolist() == [True, True, True, True, False]


def pin_classify_depth0(cmp):
    ref = {"path": np.zeros((3, 1), np.int32), "rec_a": np.zeros((3, 1, 1)),
           "rec_thr": np.ones((3, 1, 1))}
    c = cmp.classify_paths(np.zeros((3, 1), np.int32), ref, 0)
    assert c["mismatches"] == 0 and c["tokens_ok"].all()
    dev = np.zeros((3, 1), np.int32)
    dev[1, 0] = 1
    c = cmp.classify_paths(dev, ref, 0)
    assert c["bad"] == [(1, 0, None)]


def pin_classify_identical(cmp):
    ref, _, D = _ref_d3()
    c = cmp.classify_paths(ref["path"].copy(), ref, D)
    assert c["mismatches"] == 0 and c["flips_near_tie"] == 0 and c["tokens_ok"].all()


def _forced_rec(leaf, a, thr, D):
    """Records of one token, one tree, along `leaf`: heap nodes walked from
    the leaf's bits, logits and thresholds as given."""
    nodes = [0]
    for lvl in range(D):
        nodes.append(2 * nodes[-1] + 1 + ((leaf >> (D - 1 - lvl)) & 1))
    return {"rec_node": np.array(nodes, np.int32).reshape(1, 1, D + 1),
            "rec_a": np.array(a, float).reshape(1, 1, D + 1),
            "rec_thr": np.array(thr, float).reshape(1, 1, D + 1)}


def pin_path_signs(cmp):
    D = 3
    leaf = 0b110  # right, right, left
    path = np.array([[leaf]])
    # consistent signs (the leaf's own logit is unused)
    assert cmp.check_path_signs(path, _forced_rec(leaf, [2.0, 3.0, -1.0, -7.0], [1, 1, 1, 1], D), D) == []
    # level 1 went right on a clearly negative logit
    assert cmp.check_path_signs(path, _forced_rec(leaf, [2.0, -3.0, -1.0, 0], [1, 1, 1, 1], D), D) == [(0, 0, 1)]
    # ... allowed when that logit is a near-tie
    assert cmp.check_path_signs(path, _forced_rec(leaf, [2.0, -0.5, -1.0, 0], [1, 1, 1, 1], D), D) == []
    # level 2 went left on a positive logit
    assert cmp.check_path_signs(path, _forced_rec(leaf, [2.0, 3.0, 4.0, 0], [1, 1, 1, 1], D), D) == [(0, 0, 2)]
    # an exact zero lies inside the band even with a zero threshold (zero
    # weights), so either branch passes; the library's own tie rule (zero
    # goes right) is checked directly by the GPU tests on all-zero weights
    assert cmp.check_path_signs(path, _forced_rec(leaf, [0.0, 0.0, -1.0, 0], [0, 0, 0, 0], D), D) == []
    left = 0b010
    assert cmp.check_path_signs(np.array([[left]]), _forced_rec(left, [0.0, 0.0, -1.0, 0], [0, 0, 0, 0], D), D) == []
    # the band has the threshold's width: |a| = 1e-9 against a zero threshold fails
    assert cmp.check_path_signs(np.array([[left]]), _forced_rec(left, [1e-9, 0.0, -1.0, 0], [0, 0, 0, 0], D), D) == [(0, 0, 0)]
    # a leaf outside the tree
    assert cmp.check_path_signs(np.array([[8]]), _forced_rec(0, [1, 1, 1, 1], [1, 1, 1, 1], D), D) == [(0, 0, -1)]


def pin_path_signs_pruned(cmp):
    D = 2
    # one tree; leaves 0 and 1 pruned, so the root's left child (node 1) is dead
    leaf_alive = np.array([[0, 0, 1, 1]])
    alive = cmp.node_alive_from_leaves(leaf_alive, D)
    assert alive.tolist() == [[True, False, True, False, False, True, True]]
    # root logit negative (prefers the dead left child): going right is forced
    assert cmp.check_path_signs(np.array([[0b10]]), _forced_rec(0b10, [-3.0, -1.0, 0], [1, 1, 1], D), D, alive) == []
    # following the sign into the dead child is a violation
    assert cmp.check_path_signs(np.array([[0b00]]), _forced_rec(0b00, [-3.0, -1.0, 0], [1, 1, 1], D), D, alive) != []
    # a near-tie at the root allows either branch by sign, but never a dead child
    assert cmp.check_path_signs(np.array([[0b00]]), _forced_rec(0b00, [0.5, -1.0, 0], [1, 1, 1], D), D, alive) == [(0, 0, 0), (0, 0, 1)]
    # below an alive node both children alive: the sign rule applies again
    assert cmp.check_path_signs(np.array([[0b11]]), _forced_rec(0b11, [-3.0, -2.0, 0], [1, 1, 1], D), D, alive) == [(0, 0, 1)]


def pin_y_error_values(cmp):
    # y_ref = [3, 4]: rms = sqrt(12.5); element 1 off by 0.1 -> 0.1 / max(4, rms) = 0.025;
    # only element 1 is at least the rms; row norm 5 -> normwise 0.02.
    e = cmp.y_error(np.array([[3.0, 4.1]]), np.array([[3.0, 4.0]]))
    _close(e["err"], 0.025)
    _close(e["err_unfloored"], 0.025)
    _close(e["normwise"], 0.02)
    assert e["rows"] == 1
    # floor: y_ref = [0, 1], rms = sqrt(0.5); element 0 off by 0.01 -> 0.01 / sqrt(0.5)
    e = cmp.y_error(np.array([[0.01, 1.0]]), np.array([[0.0, 1.0]]))
    _close(e["err"], 0.01 / math.sqrt(0.5))
    _close(e["err_unfloored"], 0.0)
    _close(e["normwise"], 0.01)
    # negative values are compared by magnitude: y_ref = [-2, 1], off by 0.1 -> 0.1 / 2
    e = cmp.y_error(np.array([[-2.1, 1.0]]), np.array([[-2.0, 1.0]]))
    _close(e["err"], 0.05)
    # a zero reference row: absolute error
    e = cmp.y_error(np.array([[0.5, 0.0]]), np.array([[0.0, 0.0]]))
    _close(e["err"], 0.5)
    _close(e["normwise"], 0.5)
    # the row RMS is per token, not per column
    e = cmp.y_error(np.array([[1.0, 1.0], [100.0, 101.0]]), np.array([[1.0, 1.0], [100.0, 100.0]]))
    _close(e["err"], 0.01)


def pin_y_error_rows(cmp):
    ref = np.ones((3, 2))
    dev = ref.copy()
    dev[1] = 9.0
    _close(cmp.y_error(dev, ref)["err"], 8.0)
    e = cmp.y_error(dev, ref, np.array([True, False, True]))
    assert e["err"] == 0.0 and e["rows"] == 2
    e = cmp.y_error(dev, ref, np.array([False, False, False]))
    assert e["err"] == 0.0 and e["rows"] == 0
    try:
        cmp.y_error(dev[:2], ref)
    except ValueError:
        pass
    else:
        raise AssertionError("mismatched shapes must be rejected")


ALL_PINS = [pin_parting_level, pin_classify_cases, pin_classify_negative_leaf, pin_classify_depth0,
            pin_classify_identical, pin_path_signs, pin_path_signs_pruned, pin_y_error_values,
            pin_y_error_rows]
