"""Static path pruning on the GPU against the oracle's pruned mode (a leaf
mask per tree; a routed step into a subtree with no alive leaf goes to the
sibling), through fff_prune_prepare and fff_forward_pruned, on every
algorithm.  Same bars as the unpruned parity tests.
"""
import numpy as np
import pytest
import torch

import workloads
import sparse_tree_structured_amd as fff
from gpu_helpers import check, to_device, to_f64

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


def random_mask(rng, P, D, frac):
    m = (rng.random((P, 1 << D)) >= frac).astype(np.uint8)
    m[np.arange(P), rng.integers(0, 1 << D, size=P)] = 1  # every tree keeps a leaf
    return m


def subtree_mask(P, D, dead_nodes):
    """Leaves below the given heap nodes pruned, in every tree."""
    m = np.ones((P, 1 << D), np.uint8)
    for n in dead_nodes:
        level = int(np.floor(np.log2(n + 1)))
        span = 1 << (D - level)
        first = (n - ((1 << level) - 1)) * span
        m[:, first:first + span] = 0
    return m


def run_pruned(inp, mask, algo="auto", split_level=-1, chunk_tokens=0, variant=0):
    T = to_device(inp)
    s = inp.shape
    print(f"[gpu] pruned {s} algo={algo} k={split_level} alive={mask.mean():.2f}", flush=True)
    plan_T = s.T if s.T > 64 or algo == "decode" else 65536
    pr, table = fff.prune_prepare(mask, T["W_node"], T["V_node"], algo=algo,
                                  split_level=split_level, chunk_tokens=chunk_tokens, T=plan_T)
    y, path = fff.forward_pruned(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"], pr,
                                 algo=algo, split_level=split_level, chunk_tokens=chunk_tokens,
                                 variant=variant)
    torch.cuda.synchronize()
    del table
    return to_f64(y), path.cpu().numpy()


CASES = [
    # T, d, P, D, h, dtype, algo, split_level, pruned fraction
    (200, 37, 3, 4, 5, "f32", "generic", -1, 0.5),
    (150, 64, 4, 6, 16, "bf16", "generic", -1, 0.8),
    (1000, 128, 3, 4, 64, "bf16", "prefill", -1, 0.5),     # dense, ragged T
    (700, 256, 8, 6, 128, "bf16", "prefill", -1, 0.3),
    (700, 256, 8, 6, 128, "bf16", "prefill", -1, 0.9),     # a few paths left
    (500, 256, 40, 7, 64, "bf16", "prefill", -1, 0.6),     # trees packed across many tiles
    (400, 256, 3, 6, 64, "bf16", "prefill", 3, 0.5),       # token-tile deep levels
    (1100, 256, 9, 6, 128, "bf16", "prefill", 3, 0.7),     # ragged tiles and tree groups
    (300, 512, 4, 9, 64, "bf16", "prefill", 6, 0.7),
    (9, 256, 8, 5, 64, "bf16", "decode", -1, 0.5),
    (64, 1024, 16, 7, 64, "bf16", "decode", -1, 0.7),
    (3, 256, 2, 15, 256, "bf16", "decode", -1, 0.95),
]


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_pruned_shapes(case):
    T, d, P, D, h, dt, algo, k, frac = case
    inp = workloads.random_inputs(T, d, P, D, h, dt, seed=31, unit_rms_x=True)
    mask = random_mask(np.random.default_rng(T + D), P, D, frac)
    y, path = run_pruned(inp, mask, algo=algo, split_level=k)
    assert mask[np.arange(P)[None, :], path].all(), "every path ends at an alive leaf"
    check(inp, y, path, leaf_alive=mask)


@needs_gpu
def test_pruned_bucketed_deep_levels():
    # Bucketing (an explicit chunk) on pruned trees.
    inp = workloads.random_inputs(400, 256, 3, 6, 64, "bf16", seed=35, unit_rms_x=True)
    mask = random_mask(np.random.default_rng(9), 3, 6, 0.5)
    y, path = run_pruned(inp, mask, algo="prefill", split_level=3, chunk_tokens=256)
    check(inp, y, path, leaf_alive=mask)


@needs_gpu
@pytest.mark.parametrize("algo,k", [("generic", -1), ("prefill", -1), ("prefill", 3),
                                    ("decode", -1)])
def test_single_alive_leaf(algo, k):
    # One alive leaf per tree: every token takes it; y as the oracle's.
    T = 40 if algo == "decode" else 300
    inp = workloads.random_inputs(T, 256, 8, 6, 64, "bf16", seed=32, unit_rms_x=True)
    rng = np.random.default_rng(5)
    leaf = rng.integers(0, 64, size=8)
    mask = np.zeros((8, 64), np.uint8)
    mask[np.arange(8), leaf] = 1
    y, path = run_pruned(inp, mask, algo=algo, split_level=k)
    assert (path == leaf[None, :]).all()
    check(inp, y, path, leaf_alive=mask)


@needs_gpu
@pytest.mark.parametrize("algo", ["generic", "prefill", "decode"])
def test_all_alive_equals_unpruned(algo):
    # An all-alive table runs the packed / flagged code paths and must give
    # the unpruned result bit for bit.
    T = 64 if algo == "decode" else 500
    inp = workloads.random_inputs(T, 256, 8, 6, 128, "bf16", seed=33, unit_rms_x=True)
    Td = to_device(inp)
    y0, p0 = fff.forward(Td["x"], Td["W_node"], Td["b_node"], Td["V_node"], Td["W_out"], algo=algo)
    y1, p1 = run_pruned(inp, np.ones((8, 64), np.uint8), algo=algo)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(p0.cpu().numpy(), p1)
    np.testing.assert_array_equal(to_f64(y0), y1)


@needs_gpu
def test_pruned_headline_shape():
    # The OPT-1.3B-shaped depth-6 layer with half of the paths pruned at
    # random (paths and y of every token).
    inp = workloads.workload("opt1p3b_d6")
    mask = random_mask(np.random.default_rng(7), 32, 6, 0.5)
    y, path = run_pruned(inp, mask)
    check(inp, y, path, leaf_alive=mask)


@needs_gpu
@pytest.mark.parametrize("name", ["decode_skew_t64", "decode_skew_t8"])
def test_decode_skew_static(name):
    # The skewed decode workload raises the biases of heap nodes 3 and 5, so
    # the subtrees of their left children (7 and 11) see almost no tokens:
    # pruning them statically must agree with the oracle's pruned mode.
    inp = workloads.workload(name)
    mask = subtree_mask(32, 6, (7, 11))
    y, path = run_pruned(inp, mask, algo="decode")
    check(inp, y, path, leaf_alive=mask)


@needs_gpu
def test_pruned_post_variant():
    inp = workloads.random_inputs(600, 256, 8, 6, 128, "bf16", seed=34, unit_rms_x=True)
    mask = random_mask(np.random.default_rng(8), 8, 6, 0.5)
    y, path = run_pruned(inp, mask, variant=1)
    check(inp, y, path, leaf_alive=mask, variant=1)
