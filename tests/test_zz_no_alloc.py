"""fff_forward_static (the allocation-free entry point) against fff_forward
with a caller workspace: the same kernels, so y and path_out must agree bit
for bit; both are also checked against the oracle.  Two calls in a row on
one GPU, the second with fewer tokens, so the second call runs on the
region the first one left behind."""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import check, to_device, to_f64
import sparse_tree_structured_amd as fff

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")

CASES = [
    # T first, T second, d, P, D, h, algo
    ((64, 7), 2048, 32, 6, 128, "decode"),     # the decode workload's shape
    ((300, 100), 256, 8, 6, 128, "prefill"),   # every level dense, a ragged tile
    # the direct-to-LDS projection on K-blocked H, then (1000 tokens: too few
    # output tiles) the register-staged one on row-major H in the same region
    ((4096, 1000), 1024, 8, 6, 64, "prefill"),
    ((200, 50), 96, 3, 4, 24, "generic"),
]


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[f"{c[-1]}-T{c[0][0]}" for c in CASES])
def test_static_matches_workspace_forward(case):
    Ts, d, P, D, h, algo = case
    big = workloads.random_inputs(Ts[0], d, P, D, h, "bf16", seed=70 + D, unit_rms_x=True)
    dev = to_device(big)
    for T in Ts:
        x = dev["x"][:T].contiguous()
        y = torch.empty((T, d), dtype=x.dtype, device=x.device)
        path = torch.empty((T, P), dtype=torch.int32, device=x.device)
        print(f"[gpu] static forward T={T} d={d} P={P} D={D} h={h} algo={algo}", flush=True)
        fff.forward_static(x, dev["W_node"], dev["b_node"], dev["V_node"], dev["W_out"], y, path,
                           algo=algo)
        y_ref, p_ref = fff.forward(x, dev["W_node"], dev["b_node"], dev["V_node"], dev["W_out"],
                                   algo=algo)
        torch.cuda.synchronize()
        assert torch.equal(path, p_ref)
        assert torch.equal(y, y_ref)
        print(T, check(big.subset_tokens(np.arange(T)), to_f64(y), path.cpu().numpy()))
