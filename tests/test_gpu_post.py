"""FFF-post (GELU on each tree's summed output instead of on every node's
logit; explainer page, section 3.C) against the oracle's variant 1, on every
algorithm, through the C ABI on the GPU.

Same bars as the FFF parity tests: paths bit-exact except counted near-ties,
y within 1e-4 (fp32) or 2e-2 (bf16) relative error floored at the row RMS.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import check, run, to_device, to_f64
from oracle.compare import y_error

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
POST = 1


@functools.lru_cache(maxsize=None)
def wl(name):
    return workloads.workload(name)


CASES = [
    # T, d, P, D, h, dtype, algo, split_level
    (50, 37, 3, 3, 5, "f32", "generic", -1),
    (129, 96, 5, 2, 24, "f32", "generic", -1),
    (1, 1, 1, 0, 1, "f32", "generic", -1),
    (50, 37, 3, 3, 5, "bf16", "generic", -1),
    (1000, 128, 3, 4, 64, "bf16", "prefill", -1),   # every level dense, ragged T
    (333, 192, 2, 7, 128, "bf16", "prefill", -1),
    (100, 128, 2, 3, 512, "bf16", "prefill", -1),   # widest node output
    (257, 256, 2, 6, 256, "bf16", "prefill", -1),
    (400, 256, 3, 6, 64, "bf16", "prefill", 3),     # bucketed deep levels
    (300, 512, 4, 9, 64, "bf16", "prefill", 6),
    (77, 256, 4, 10, 64, "bf16", "auto", -1),       # deep trees
    (1, 256, 2, 0, 256, "bf16", "decode", -1),
    (17, 512, 8, 5, 64, "bf16", "decode", -1),
    (33, 768, 4, 9, 128, "bf16", "decode", -1),
    (64, 1024, 16, 7, 64, "bf16", "decode", -1),
]


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_post_shapes(case):
    T, d, P, D, h, dt, algo, k = case
    inp = workloads.random_inputs(T, d, P, D, h, dt, seed=21, unit_rms_x=True)
    y, path = run(inp, algo=algo, split_level=k, variant=POST)
    check(inp, y, path, variant=POST)


@needs_gpu
@pytest.mark.parametrize("name", ["gpt125m", "opt1p3b_d6", "decode_skew_t64"])
def test_post_workloads(name):
    inp = wl(name)
    y, path = run(inp, variant=POST)
    check(inp, y, path, variant=POST)


@needs_gpu
def test_post_routes_like_fff_and_differs_in_y():
    # The variant moves the GELU only: identical paths, different outputs.
    inp = wl("gpt125m")
    y0, p0 = run(inp, variant=0)
    y1, p1 = run(inp, variant=POST)
    np.testing.assert_array_equal(p0, p1)
    assert np.abs(y0 - y1).max() > 1e-2 * np.sqrt(np.mean(y0 ** 2))


@needs_gpu
@pytest.mark.parametrize("algo", ["generic", "prefill"])
def test_post_route_h_elementwise(algo):
    # fff_route's H against the oracle's H element by element: the GELU sits
    # on each element of H, so this checks it where it is applied.
    import sparse_tree_structured_amd as fff
    inp = workloads.random_inputs(300, 256, 4, 5, 64, "bf16", seed=22, unit_rms_x=True)
    T = to_device(inp)
    print(f"[gpu] route post algo={algo}", flush=True)
    H, path = fff.route(T["x"], T["W_node"], T["b_node"], T["V_node"], algo=algo, variant=POST)
    torch.cuda.synchronize()
    f = inp.as_f64()
    ref = oracle.forward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"], want_y=False,
                         want_H=True, want_records=True, variant=POST)
    path = path.cpu().numpy()
    ok = (path == ref["path"]).all(axis=1)
    assert ok.mean() > 0.99
    # bf16 H: one rounding of a value computed in fp32 (relative 2^-8), floored
    # at the row RMS like y.
    err = y_error(to_f64(H)[ok], ref["H"][ok])
    assert err["err"] <= 1e-2, err
