"""Seeded synthetic inputs for the Fast FeedForward (FFF) layer forward pass.

This module is shared by the tests, the benchmark and the smoke check, and by
nothing else.  It draws random numbers and rounds them to the storage dtype;
it holds none of the layer's arithmetic (no logits, routing, GELU or
projection).  Both the CPU oracle and the HIP library consume what it makes.

Random numbers
--------------
A counter-based splitmix64 stream: the 64-bit word for counter value ``c``
under key ``k`` is ``mix64(k + (c + 1) * GOLDEN)``, with ``mix64`` the
splitmix64 finaliser (Steele, Lea, Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014).  The key packs (seed, tensor id); tensor ids are
x=0, W_node=1, b_node=2, V_node=3, W_out=4.  Element ``i`` of a tensor takes the
uniforms of counters ``2i`` and ``2i+1`` and turns them into one standard
normal by the Box-Muller transform in float64.  A normal of variance ``s`` is
``sqrt(s)`` times that draw.

Rounding
--------
Values are generated in float64 and rounded once, round-to-nearest-even, to
the storage dtype (IEEE float32, or bfloat16 kept as its raw uint16 bits).

Layer shapes and layouts (all row-major, contiguous)
-----------------------------------------------------
The FFF paper's explainer page ("Dynamic sparsity in tree-structured
feed-forward layers at scale", gist.science, section 2) describes P parallel
perfect binary trees of depth D; each tree here has N = 2**(D+1) - 1 nodes in
heap order (root 0, children of n at 2n+1 and 2n+2).

    x      [T, d]          W_node [P, N, d]     b_node [P, N]
    V_node [P, N, h]       W_out  [P*h, d]

Workloads
---------
``tiny``        T=64, d=64, P=2, D=3, h=32, float32.
``gpt125m``     T=8192 (8 x 1024), d=768, P=16, D=5, h=64, bf16.
``opt1p3b_d4``  T=16384 (8 x 2048), d=2048, P=32, D=4, h=128, bf16.
``opt1p3b_d6``  T=16384, d=2048, P=32, D=6, h=128, bf16.
``decode_skew`` T in {1, 8, 64}, d=2048, P=32, D=6, h=128, bf16; x is the
                first T rows of one 64-row draw, and the bias of heap nodes 3
                and 5 (level 2, positions 0 and 2) of every tree is raised by
                3 * ||w_n||_2, so those nodes almost always route right and
                their left subtrees receive no tokens.

Distributions: x ~ N(0, 1) (for the OPT-shaped workloads each row is then
rescaled in float64 to unit RMS before rounding); w_n ~ N(0, 1/d);
b_n ~ N(0, 0.01); v_n ~ N(0, 1/h); W_out ~ N(0, 1/(P*h)).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_IDS = {"x": 0, "W_node": 1, "b_node": 2, "V_node": 3, "W_out": 4}

# Element counts above this are generated in slices to bound host memory.
_CHUNK = 1 << 22


def _mix64(z: np.ndarray) -> np.ndarray:
    """splitmix64 finaliser on a uint64 array (wrapping arithmetic)."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, tensor_id: int) -> np.uint64:
    return np.uint64(((int(seed) & 0xFFFFFFFF) << 24) ^ ((int(tensor_id) & 0xFF) << 16) ^ 0x5EED)


def uniform_words(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    """Raw 64-bit words for counters start .. start+count-1."""
    with np.errstate(over="ignore"):
        c = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        return _mix64(_key(seed, tensor_id) + c * GOLDEN)


def standard_normal(seed: int, tensor_id: int, n: int) -> np.ndarray:
    """n standard normal float64 draws for (seed, tensor id), Box-Muller."""
    out = np.empty(n, dtype=np.float64)
    scale = 1.0 / 9007199254740992.0  # 2**-53
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        w = uniform_words(seed, tensor_id, 2 * s, 2 * m)
        # (0, 1] for the log argument, [0, 1) for the angle.
        u1 = ((w[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * scale
        u2 = (w[1::2] >> np.uint64(11)).astype(np.float64) * scale
        out[s:s + m] = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
    return out


def round_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16, nearest-even, in one step.

    bfloat16 keeps 8 significant bits and float32's exponent range.  For a
    value with binary exponent e (v = m * 2**e, 0.5 <= |m| < 1) the spacing of
    bfloat16 numbers is 2**(e-8), floored at the subnormal spacing 2**-133.
    Dividing by a power of two is exact in float64, and numpy's rint rounds
    half to even, so q * spacing is the correctly rounded bfloat16 value.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q_exp = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -q_exp)), q_exp)
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)  # exact: r is representable in bfloat16
    bits = f.view(np.uint32)
    return (bits >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bits to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class Shape:
    T: int
    d: int
    P: int
    D: int
    h: int
    dtype: str  # "f32" or "bf16"

    @property
    def N(self) -> int:
        return (1 << (self.D + 1)) - 1


@dataclasses.dataclass
class Inputs:
    """One layer's inputs in storage form.

    For dtype "bf16" every array is uint16 holding bfloat16 bits; for "f32"
    every array is float32.
    """
    shape: Shape
    x: np.ndarray
    W_node: np.ndarray
    b_node: np.ndarray
    V_node: np.ndarray
    W_out: np.ndarray

    def as_f64(self) -> Dict[str, np.ndarray]:
        """Exact float64 copies of every tensor (for the oracle)."""
        conv = bf16_bits_to_f64 if self.shape.dtype == "bf16" else (lambda a: a.astype(np.float64))
        return {k: conv(getattr(self, k)) for k in ("x", "W_node", "b_node", "V_node", "W_out")}

    def subset_tokens(self, idx: np.ndarray) -> "Inputs":
        s = dataclasses.replace(self.shape, T=int(len(idx)))
        return Inputs(s, self.x[idx], self.W_node, self.b_node, self.V_node, self.W_out)


def _store(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16_bits(v)
    if dtype == "f32":
        return v.astype(np.float32)
    raise ValueError(dtype)


def _normal(seed: int, name: str, shape, var: float) -> np.ndarray:
    n = int(np.prod(shape))
    return (math.sqrt(var) * standard_normal(seed, TENSOR_IDS[name], n)).reshape(shape)


def _bf16_or_f32_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)


def make_inputs(shape: Shape, seed: int = 0, unit_rms_x: bool = False,
                skew_nodes: Optional[tuple] = None, skew_sigmas: float = 3.0,
                x_rows_drawn: Optional[int] = None) -> Inputs:
    """Draw one layer's inputs.

    unit_rms_x   rescale each x row to RMS 1 (float64) before rounding.
    skew_nodes   heap node ids whose bias is raised by skew_sigmas*||w_n||_2
                 (norm of the rounded weight row) in every tree.
    x_rows_drawn draw this many x rows and keep the first T (so smaller
                 batches are prefixes of a larger one).
    """
    T, d, P, D, h, dt = shape.T, shape.d, shape.P, shape.D, shape.h, shape.dtype
    N = shape.N
    rows = T if x_rows_drawn is None else int(x_rows_drawn)
    assert rows >= T
    x = _normal(seed, "x", (rows, d), 1.0)[:T]
    if unit_rms_x and T > 0:
        rms = np.sqrt(np.mean(x * x, axis=1, keepdims=True))
        x = x / rms
    W = _store(_normal(seed, "W_node", (P, N, d), 1.0 / d), dt)
    b = _normal(seed, "b_node", (P, N), 0.01)
    if skew_nodes:
        Wf = _bf16_or_f32_to_f64(W, dt)
        for n in skew_nodes:
            if n < N:
                b[:, n] += skew_sigmas * np.sqrt(np.sum(Wf[:, n, :] ** 2, axis=1))
    V = _normal(seed, "V_node", (P, N, h), 1.0 / h)
    Wo = _normal(seed, "W_out", (P * h, d), 1.0 / (P * h))
    return Inputs(shape, _store(x, dt), W, _store(b, dt), _store(V, dt), _store(Wo, dt))


# Named workloads.  Each maps to (shape, generator options).
WORKLOADS = {
    "tiny": (Shape(64, 64, 2, 3, 32, "f32"), {}),
    "gpt125m": (Shape(8192, 768, 16, 5, 64, "bf16"), {}),
    "opt1p3b_d4": (Shape(16384, 2048, 32, 4, 128, "bf16"), {"unit_rms_x": True}),
    "opt1p3b_d6": (Shape(16384, 2048, 32, 6, 128, "bf16"), {"unit_rms_x": True}),
    "decode_skew_t1": (Shape(1, 2048, 32, 6, 128, "bf16"),
                       {"unit_rms_x": True, "skew_nodes": (3, 5), "x_rows_drawn": 64}),
    "decode_skew_t8": (Shape(8, 2048, 32, 6, 128, "bf16"),
                       {"unit_rms_x": True, "skew_nodes": (3, 5), "x_rows_drawn": 64}),
    "decode_skew_t64": (Shape(64, 2048, 32, 6, 128, "bf16"),
                        {"unit_rms_x": True, "skew_nodes": (3, 5), "x_rows_drawn": 64}),
}


def workload(name: str, seed: int = 0) -> Inputs:
    shape, opts = WORKLOADS[name]
    return make_inputs(shape, seed=seed, **opts)


def random_inputs(T: int, d: int, P: int, D: int, h: int, dtype: str = "bf16",
                  seed: int = 0, **opts) -> Inputs:
    """Inputs of any shape with the workloads' distributions."""
    return make_inputs(Shape(T, d, P, D, h, dtype), seed=seed, **opts)
