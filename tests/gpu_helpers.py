"""Helpers for the GPU parity tests: upload generator output, run the library,
check against the oracle.

``check`` compares every token:
* paths (t, p) by (t, p): bit-exact except near-tie flips, which are counted;
* each flipped token again, with the oracle forced along the device's own
  paths: every decision on them must follow its logit's sign (or be a
  near-tie), and the token's y must match the oracle's y along those paths;
* y of every other token against the oracle's own y.
"""
from __future__ import annotations

import hashlib
from typing import Dict, Optional

import numpy as np
import torch

import oracle
from oracle.compare import check_path_signs, classify_paths, node_alive_from_leaves, y_error
import sparse_tree_structured_amd as fff

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_device(inp, dev="cuda:0"):
    out = {}
    for k in ("x", "W_node", "b_node", "V_node", "W_out"):
        a = getattr(inp, k)
        if inp.shape.dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a))
        out[k] = t.to(dev)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run(inp, algo="auto", split_level=-1, dev="cuda:0", variant=0, chunk_tokens=0,
        plan_flags=0):
    T = to_device(inp, dev)
    print(f"[gpu] forward {inp.shape} algo={algo} k={split_level} variant={variant} "
          f"flags={plan_flags}", flush=True)
    y, path = fff.forward(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"], algo=algo,
                          split_level=split_level, chunk_tokens=chunk_tokens, variant=variant,
                          plan_flags=plan_flags)
    torch.cuda.synchronize()
    return to_f64(y), path.cpu().numpy()


# The oracle's natural-route result for an input set, by content: the same
# workload is checked under several plans, and the oracle's answer does not
# depend on the plan.
_REF_CACHE: Dict[str, Dict[str, np.ndarray]] = {}


def _key(inp, variant, leaf_alive) -> str:
    h = hashlib.blake2b(digest_size=16)
    for k in ("x", "W_node", "b_node", "V_node", "W_out"):
        a = np.ascontiguousarray(getattr(inp, k))
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    h.update(f"{inp.shape.dtype}|{variant}".encode())
    if leaf_alive is not None:
        h.update(np.ascontiguousarray(leaf_alive, dtype=np.uint8).tobytes())
    return h.hexdigest()


def reference(inp, variant=0, leaf_alive=None, nthreads=None):
    key = _key(inp, variant, leaf_alive)
    if key not in _REF_CACHE:
        if len(_REF_CACHE) >= 4:
            _REF_CACHE.pop(next(iter(_REF_CACHE)))
        f = inp.as_f64()
        _REF_CACHE[key] = oracle.forward(f["x"], f["W_node"], f["b_node"], f["V_node"],
                                         f["W_out"], want_y=True, want_records=True,
                                         nthreads=nthreads, variant=variant,
                                         leaf_alive=leaf_alive)
    return _REF_CACHE[key]


def check(inp, y_dev, path_dev, sample=None, nthreads=None, max_flip_frac=1e-3, variant=0,
          leaf_alive=None):
    """Paths and y of every token against the oracle (``sample`` restricts
    the y comparison to those rows; the tests pass None).  Returns a summary
    dict; raises AssertionError on failure."""
    s = inp.shape
    ref = reference(inp, variant, leaf_alive, nthreads)
    cls = classify_paths(path_dev, ref, s.D)
    assert not cls["bad"], f"routing mismatches beyond near-ties: {cls['bad'][:5]}"
    assert cls["flips_near_tie"] <= max(2, max_flip_frac * s.T * s.P), cls["flips_near_tie"]
    tol = TOL[s.dtype]
    rows = np.arange(s.T) if sample is None else np.asarray(sample)
    ok = rows[cls["tokens_ok"][rows]]
    err = y_error(y_dev[ok], ref["y"][ok])
    assert err["err"] <= tol, f"y error {err} above {tol}"
    flipped = rows[~cls["tokens_ok"][rows]]
    err_f = {"err": 0.0, "rows": 0}
    if len(flipped):
        f = inp.as_f64()
        fr = oracle.forward(f["x"][flipped], f["W_node"], f["b_node"], f["V_node"], f["W_out"],
                            forced=np.ascontiguousarray(path_dev[flipped], dtype=np.int32),
                            want_y=True, want_records=True, nthreads=nthreads, variant=variant)
        alive = node_alive_from_leaves(leaf_alive, s.D) if leaf_alive is not None else None
        viol = check_path_signs(path_dev[flipped], fr, s.D, alive)
        assert not viol, f"device paths of flipped tokens break the sign rule: {viol[:5]}"
        err_f = y_error(y_dev[flipped], fr["y"])
        assert err_f["err"] <= tol, f"y error of flipped tokens {err_f} above {tol}"
    return {"flips": cls["flips_near_tie"], "tokens_flipped": int(len(flipped)),
            "y_err": err["err"], "y_err_flipped": err_f["err"], "rows": int(len(rows))}


def sample_rows(T, n=96, seed=0):
    rng = np.random.default_rng(seed)
    picks = set([0, T - 1, T // 2]) | set(rng.integers(0, T, size=n).tolist())
    return np.array(sorted(picks))
