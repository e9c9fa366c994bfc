"""CPU oracle for the Fast FeedForward (FFF) layer forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The HIP library
(``sparse_tree_structured_amd``) never does, and shares no code with it.

The arithmetic lives in ``fff_oracle.c`` (plain C, float64, OpenMP over
tokens).  This module compiles it with gcc on first use (or when
``build()`` is called) and marshals numpy arrays through ctypes.

Parity pins for every function here are in ``tests/test_oracle_pins.py``:
brute-force enumeration of all root-to-leaf paths on tiny trees, hand-built
weights whose routing is known, the all-zero tie case, the constant-bias
closed form, the depth-0 reduction to a dense one-hidden-layer MLP, the
visit count against the paper's Table 4 sparsity column, and invariances.
``tests/test_oracle_mutants.py`` plants plausible mistakes in a copy of the C
source and checks that some pin catches each one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "fff_oracle.c")
LIBRARY = os.path.join(_HERE, "libfff_oracle.so")

CFLAGS = ["-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-shared", "-fPIC"]


def compile_oracle(source: str, out: str) -> str:
    """Compile an oracle C source into a shared library."""
    cmd = ["gcc", *CFLAGS, "-o", out, source, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def build() -> str:
    """(Re)compile the oracle library next to its source."""
    tmp = LIBRARY + ".tmp"
    compile_oracle(SOURCE, tmp)
    os.replace(tmp, LIBRARY)
    return LIBRARY


_LIBS: Dict[str, ctypes.CDLL] = {}


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the oracle library (building it first if it is missing or stale)."""
    if path is None:
        path = LIBRARY
        if (not os.path.exists(path)) or os.path.getmtime(path) < os.path.getmtime(SOURCE):
            build()
    if path in _LIBS:
        return _LIBS[path]
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    up = ctypes.POINTER(ctypes.c_uint8)
    lib.fffo_forward.restype = ctypes.c_int
    lib.fffo_forward.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, ip, up, dp, dp, ip,
                                 dp, dp, ip, ctypes.c_int]
    lib.fffo_backward.restype = ctypes.c_int
    lib.fffo_backward.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, up, dp, dp, dp,
                                  dp, dp, dp, ctypes.c_int]
    _LIBS[path] = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _dptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def forward(x: np.ndarray, W_node: np.ndarray, b_node: np.ndarray, V_node: np.ndarray,
            W_out: np.ndarray, forced: Optional[np.ndarray] = None, want_y: bool = True,
            want_H: bool = False, want_records: bool = False, variant: int = 0,
            leaf_alive: Optional[np.ndarray] = None,
            nthreads: Optional[int] = None, lib: Optional[ctypes.CDLL] = None) -> Dict[str, np.ndarray]:
    """Run the oracle.

    Arrays are float64 (widened exactly from the storage dtype):
    x [T,d], W_node [P,N,d], b_node [P,N], V_node [P,N,h], W_out [P*h,d].
    ``forced`` [T,P] int32 leaf indices walks those paths instead of routing.
    ``variant`` 0 is FFF (GELU on each node's logit before the sum), 1 is
    FFF-post (GELU applied once to each tree's summed h-vector).
    ``leaf_alive`` [P, 2^D] (nonzero = alive) prunes paths statically: a
    routed step into a subtree with no alive leaf goes to the sibling.

    Returns a dict with ``path`` [T,P] int32, and as requested ``y`` [T,d],
    ``H`` [T,P*h], and the per-visit records ``rec_a``, ``rec_thr`` (float64)
    and ``rec_node`` (int32, heap index, -1 where nothing was recorded), each
    [T,P,D+1].
    """
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    W_node = np.ascontiguousarray(W_node, dtype=np.float64)
    b_node = np.ascontiguousarray(b_node, dtype=np.float64)
    V_node = np.ascontiguousarray(V_node, dtype=np.float64)
    W_out = np.ascontiguousarray(W_out, dtype=np.float64)
    T, d = x.shape
    P, N, d2 = W_node.shape
    h = V_node.shape[2]
    D = int(round(np.log2(N + 1))) - 1
    if d2 != d or (1 << (D + 1)) - 1 != N or b_node.shape != (P, N) or \
            V_node.shape != (P, N, h) or W_out.shape != (P * h, d):
        raise ValueError("inconsistent shapes")
    out: Dict[str, np.ndarray] = {"path": np.empty((T, P), dtype=np.int32)}
    if want_y:
        out["y"] = np.empty((T, d), dtype=np.float64)
    if want_H:
        out["H"] = np.empty((T, P * h), dtype=np.float64)
    if want_records:
        out["rec_a"] = np.full((T, P, D + 1), np.nan)
        out["rec_thr"] = np.full((T, P, D + 1), np.nan)
        out["rec_node"] = np.full((T, P, D + 1), -1, dtype=np.int32)
    if forced is not None:
        forced = np.ascontiguousarray(forced, dtype=np.int32)
        if forced.shape != (T, P):
            raise ValueError("forced must be [T,P]")
    alive_ptr = None
    if leaf_alive is not None:
        leaf_alive = np.ascontiguousarray(leaf_alive, dtype=np.uint8)
        if leaf_alive.shape != (P, 1 << D):
            raise ValueError("leaf_alive must be [P, 2^D]")
        alive_ptr = leaf_alive.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    rc = lib.fffo_forward(T, d, P, D, h, int(variant), _dptr(x), _dptr(W_node), _dptr(b_node),
                          _dptr(V_node), _dptr(W_out), _iptr(forced), alive_ptr, _dptr(out.get("y")), _dptr(out.get("H")),
                          _iptr(out["path"]), _dptr(out.get("rec_a")), _dptr(out.get("rec_thr")),
                          _iptr(out.get("rec_node")), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the shape, variant or mask")
    return out


def backward(x: np.ndarray, W_node: np.ndarray, b_node: np.ndarray, V_node: np.ndarray,
             W_out: np.ndarray, dy: np.ndarray, variant: int = 0,
             leaf_alive: Optional[np.ndarray] = None, nthreads: Optional[int] = None,
             lib: Optional[ctypes.CDLL] = None) -> Dict[str, np.ndarray]:
    """Gradients of sum(y * dy) with the forward's paths held fixed.

    Returns float64 ``dx`` [T,d], ``dW_node`` [P,N,d], ``db_node`` [P,N],
    ``dV_node`` [P,N,h] and ``dW_out`` [P*h,d].
    """
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    W_node = np.ascontiguousarray(W_node, dtype=np.float64)
    b_node = np.ascontiguousarray(b_node, dtype=np.float64)
    V_node = np.ascontiguousarray(V_node, dtype=np.float64)
    W_out = np.ascontiguousarray(W_out, dtype=np.float64)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    T, d = x.shape
    P, N, _ = W_node.shape
    h = V_node.shape[2]
    D = int(round(np.log2(N + 1))) - 1
    if dy.shape != (T, d) or W_out.shape != (P * h, d):
        raise ValueError("inconsistent shapes")
    alive_ptr = None
    if leaf_alive is not None:
        leaf_alive = np.ascontiguousarray(leaf_alive, dtype=np.uint8)
        if leaf_alive.shape != (P, 1 << D):
            raise ValueError("leaf_alive must be [P, 2^D]")
        alive_ptr = leaf_alive.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    out = {"dx": np.empty((T, d)), "dW_node": np.empty((P, N, d)), "db_node": np.empty((P, N)),
           "dV_node": np.empty((P, N, h)), "dW_out": np.empty((P * h, d))}
    rc = lib.fffo_backward(T, d, P, D, h, int(variant), _dptr(x), _dptr(W_node), _dptr(b_node),
                           _dptr(V_node), _dptr(W_out), alive_ptr, _dptr(dy), _dptr(out["dx"]),
                           _dptr(out["dW_node"]), _dptr(out["db_node"]), _dptr(out["dV_node"]),
                           _dptr(out["dW_out"]), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the shape, variant or mask")
    return out


def forward_inputs(inp, **kw) -> Dict[str, np.ndarray]:
    """Run the oracle on a ``workloads.Inputs`` (widened to float64)."""
    f = inp.as_f64()
    return forward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"], **kw)
