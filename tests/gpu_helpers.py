"""Helpers for the GPU parity tests: upload generator output, run the library,
check against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.compare import classify_paths, y_error
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


def run(inp, algo="auto", split_level=-1, dev="cuda:0", variant=0, chunk_tokens=0):
    T = to_device(inp, dev)
    print(f"[gpu] forward {inp.shape} algo={algo} k={split_level} variant={variant}", flush=True)
    y, path = fff.forward(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"], algo=algo,
                          split_level=split_level, chunk_tokens=chunk_tokens, variant=variant)
    torch.cuda.synchronize()
    return to_f64(y), path.cpu().numpy()


def check(inp, y_dev, path_dev, sample=None, nthreads=None, max_flip_frac=1e-3, variant=0,
          leaf_alive=None):
    """Paths of all tokens against the oracle, y on `sample` token rows (all
    if None).  Returns a summary dict; raises AssertionError on failure."""
    s = inp.shape
    f = inp.as_f64()
    ref = oracle.forward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"], want_y=False,
                         want_records=True, nthreads=nthreads, variant=variant,
                         leaf_alive=leaf_alive)
    cls = classify_paths(path_dev, ref, s.D)
    assert not cls["bad"], f"routing mismatches beyond near-ties: {cls['bad'][:5]}"
    assert cls["flips_near_tie"] <= max(2, max_flip_frac * s.T * s.P), cls["flips_near_tie"]
    rows = np.arange(s.T) if sample is None else np.asarray(sample)
    rows = rows[cls["tokens_ok"][rows]]
    ry = oracle.forward(f["x"][rows], f["W_node"], f["b_node"], f["V_node"], f["W_out"],
                        nthreads=nthreads, variant=variant, leaf_alive=leaf_alive)
    np.testing.assert_array_equal(ry["path"], path_dev[rows])
    err = y_error(y_dev[rows], ry["y"])
    assert err["err"] <= TOL[s.dtype], f"y error {err} above {TOL[s.dtype]}"
    return {"flips": cls["flips_near_tie"], "y_err": err["err"], "rows": len(rows)}


def sample_rows(T, n=96, seed=0):
    rng = np.random.default_rng(seed)
    picks = set([0, T - 1, T // 2]) | set(rng.integers(0, T, size=n).tolist())
    return np.array(sorted(picks))
