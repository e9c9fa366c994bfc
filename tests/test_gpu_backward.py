"""Backward pass on the GPU against the oracle's (gradients of sum(y * dy)
with the forward's paths held fixed), through fff_backward.

Every gradient is compared element by element.  Float32 layers: error =
max |g - g_ref| / max(|g_ref|, RMS of g_ref over the tensor) at most 1e-4,
and the normwise error at most 1e-4.  bf16 layers: each element must lie
within 2 u E of the oracle's value, where u = 2^-8 and E is the running-error
bound ``oracle.bounds.backward_bound`` derives, in float64 from the oracle's
own records, for a computation that rounds H, dH (dS for FFF-post), da, the
per-node weights and dx to bf16 once each and sums in float32 (its pins:
``tests/test_bound_pins.py``).  The factor 2 leaves room for the terms of
second order in u and for float32 GELU and tanh, which the bound leaves out.
Inputs are checked to route identically on both sides (no near-tie flips),
since a flipped path changes which nodes get gradient.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import bounds
import sparse_tree_structured_amd as fff
from gpu_helpers import to_device, to_f64

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
TOL_F32 = 1e-4       # f32 layers: elementwise (floored at the RMS) and normwise
BOUND_FACTOR = 2.0   # bf16 layers: |g - g_ref| <= BOUND_FACTOR * u * E
GRADS = ("dx", "dW_node", "db_node", "dV_node", "dW_out")


def grad_error(g, ref):
    g = np.asarray(g, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(g - ref) / den)) if ref.size else 0.0


def norm_error(g, ref):
    g = np.asarray(g, dtype=np.float64)
    nr = np.linalg.norm(ref)
    return float(np.linalg.norm(g - ref) / nr) if nr > 0 else float(np.linalg.norm(g))


def bound_ratio(g, ref, E):
    """max over elements of |g - g_ref| / (BOUND_FACTOR u E); at most 1 passes."""
    g = np.asarray(g, dtype=np.float64)
    lim = BOUND_FACTOR * bounds.U_BF16 * E
    diff = np.abs(g - ref)
    if not diff.size:
        return 0.0
    return float(np.max(np.where(lim > 0, diff / np.where(lim > 0, lim, 1.0),
                                 np.where(diff > 0, np.inf, 0.0))))


def assert_grads(dt, g, ref, f, dy64, rec, variant):
    """f: the float64 inputs of the tokens in g and ref; rec: their records."""
    errs = {k: (grad_error(g[k], ref[k]), norm_error(g[k], ref[k])) for k in GRADS}
    print("grad errors (elementwise, normwise)", errs, flush=True)
    if dt == "f32":
        bad = {k: e for k, e in errs.items() if e[0] > TOL_F32 or e[1] > TOL_F32}
        assert not bad, bad
        return errs
    E = bounds.backward_bound(f["x"], f["W_node"], f["V_node"], f["W_out"], dy64,
                              rec["rec_node"], rec["rec_a"], variant)
    ratios = {k: bound_ratio(g[k], ref[k], E[k]) for k in GRADS}
    print("error / (2 u E), max per gradient", ratios, flush=True)
    bad = {k: r for k, r in ratios.items() if not r <= 1.0}
    assert not bad, bad
    return ratios


def make_dy(inp, seed):
    s = inp.shape
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((s.T, s.d))
    if s.dtype == "bf16":
        t = torch.from_numpy(dy).to(torch.bfloat16)
        return t, t.double().numpy()
    t = torch.from_numpy(dy.astype(np.float32))
    return t, t.double().numpy()


def run_backward(inp, algo="auto", variant=0, seed=7):
    T = to_device(inp)
    dy_t, dy64 = make_dy(inp, seed)
    dy_t = dy_t.to(T["x"].device)
    print(f"[gpu] backward {inp.shape} algo={algo} variant={variant}", flush=True)
    g = fff.backward(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"], dy_t, algo=algo,
                     variant=variant)
    _, path = fff.forward(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"],
                          algo="generic", variant=variant)
    torch.cuda.synchronize()
    return {k: to_f64(v) for k, v in g.items()}, path.cpu().numpy(), dy64


def check_grads(inp, g, path, dy64, variant=0):
    f = inp.as_f64()
    rec = oracle.forward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"],
                         want_y=False, want_records=True, variant=variant)
    np.testing.assert_array_equal(path, rec["path"])
    ref = oracle.backward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"], dy64,
                          variant=variant)
    return assert_grads(inp.shape.dtype, g, ref, f, dy64, rec, variant)


GENERIC = [
    # T, d, P, D, h, dtype
    (50, 37, 3, 3, 5, "f32"),
    (129, 96, 5, 2, 24, "f32"),
    (1, 1, 1, 0, 1, "f32"),
    (64, 64, 2, 3, 32, "f32"),
    (40, 64, 4, 4, 16, "bf16"),
    (33, 128, 3, 6, 64, "bf16"),
]


@needs_gpu
@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("shape", GENERIC, ids=[str(s) for s in GENERIC])
def test_backward_generic(shape, variant):
    T, d, P, D, h, dt = shape
    inp = workloads.random_inputs(T, d, P, D, h, dt, seed=50 + D, unit_rms_x=True)
    g, path, dy = run_backward(inp, algo="generic", variant=variant)
    check_grads(inp, g, path, dy, variant=variant)


@needs_gpu
def test_backward_zero_tokens_zeroes_gradients():
    inp = workloads.random_inputs(4, 64, 2, 3, 32, "f32", seed=1)
    T = to_device(inp)
    x0 = T["x"][:0]
    dy0 = torch.empty((0, 64), device=x0.device)
    g = fff.backward(x0, T["W_node"], T["b_node"], T["V_node"], T["W_out"], dy0, algo="generic",
                     out={"dx": torch.empty((0, 64), device=x0.device),
                          "dW_node": torch.full(T["W_node"].shape, 7.0, device=x0.device),
                          "db_node": torch.full(T["b_node"].shape, 7.0, device=x0.device),
                          "dV_node": torch.full(T["V_node"].shape, 7.0, device=x0.device),
                          "dW_out": torch.full(T["W_out"].shape, 7.0, device=x0.device)})
    torch.cuda.synchronize()
    for k in ("dW_node", "db_node", "dV_node", "dW_out"):
        assert (g[k] == 0).all()


MFMA = [
    # T, d, P, D, h  (bf16, every level dense)
    (300, 256, 4, 6, 64),      # tokens not a multiple of the 256-token padding
    (1000, 128, 8, 2, 64),     # the shallowest dense plan (3 levels)
    (500, 512, 2, 7, 64),      # 256 columns per tree
    (257, 256, 16, 5, 128),
    (64, 192, 8, 3, 64),
]


@needs_gpu
@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("shape", MFMA, ids=[str(s) for s in MFMA])
def test_backward_mfma(shape, variant):
    T, d, P, D, h = shape
    inp = workloads.random_inputs(T, d, P, D, h, "bf16", seed=70 + D, unit_rms_x=True)
    g, path, dy = run_backward(inp, algo="prefill", variant=variant)
    check_grads(inp, g, path, dy, variant=variant)


@needs_gpu
@pytest.mark.parametrize("variant", [0, 1])
def test_backward_full_size_sampled(variant):
    # The OPT-1.3B-shaped depth-6 layer in the launch configuration the
    # benchmark times, with dy nonzero on a sample of tokens only: every
    # gradient then depends on those tokens alone, so the oracle's backward
    # over the sample is the exact reference.
    inp = workloads.workload("opt1p3b_d6")
    s = inp.shape
    T = to_device(inp)
    print(f"[gpu] backward full size variant={variant}", flush=True)
    _, path = fff.forward(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"],
                          variant=variant)
    torch.cuda.synchronize()
    path = path.cpu().numpy()
    # Sampled tokens whose paths match the oracle's (a near-tie flip would
    # move gradient to other nodes).
    cand = np.sort(np.random.default_rng(3).choice(s.T, size=48, replace=False))
    fc = inp.subset_tokens(cand).as_f64()
    ok = (oracle.forward(fc["x"], fc["W_node"], fc["b_node"], fc["V_node"], fc["W_out"],
                         want_y=False, variant=variant)["path"] == path[cand]).all(axis=1)
    rows = cand[ok][:24]
    assert len(rows) == 24
    dy = np.zeros((s.T, s.d))
    dy[rows] = np.random.default_rng(4).standard_normal((len(rows), s.d))
    dy_t = torch.from_numpy(dy).to(torch.bfloat16)
    dy64 = dy_t.double().numpy()
    g = fff.backward(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"],
                     dy_t.to(T["x"].device), variant=variant)
    torch.cuda.synchronize()
    g = {k: to_f64(v) for k, v in g.items()}
    f = inp.subset_tokens(rows).as_f64()
    ref = oracle.backward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"], dy64[rows],
                          variant=variant)
    rec = oracle.forward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"],
                         want_y=False, want_records=True, variant=variant)
    assert (g["dx"][np.setdiff1d(np.arange(s.T), rows)] == 0).all()
    g["dx"] = g["dx"][rows]
    assert_grads("bf16", g, ref, f, dy64[rows], rec, variant)
