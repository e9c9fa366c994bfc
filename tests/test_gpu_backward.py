"""Backward pass on the GPU against the oracle's (gradients of sum(y * dy)
with the forward's paths held fixed), through fff_backward.

Every gradient is compared element by element: error = max |g - g_ref| /
max(|g_ref|, RMS of g_ref over the tensor), at most 1e-4 for float32
layers and 2e-2 for bf16 ones (dx is rounded to the layer dtype; parameter
gradients are float32).  Inputs are checked to route identically on both
sides (no near-tie flips), since a flipped path changes which nodes get
gradient.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import sparse_tree_structured_amd as fff
from gpu_helpers import to_device, to_f64

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
TOL = {"f32": 1e-4, "bf16": 2e-2}
GRADS = ("dx", "dW_node", "db_node", "dV_node", "dW_out")


def grad_error(g, ref):
    g = np.asarray(g, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(g - ref) / den)) if ref.size else 0.0


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
    ref_path = oracle.forward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"],
                              want_y=False, variant=variant)["path"]
    np.testing.assert_array_equal(path, ref_path)
    ref = oracle.backward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"], dy64,
                          variant=variant)
    errs = {k: grad_error(g[k], ref[k]) for k in GRADS}
    print("grad errors", errs, flush=True)
    bad = {k: e for k, e in errs.items() if e > TOL[inp.shape.dtype]}
    assert not bad, bad
    return errs


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
