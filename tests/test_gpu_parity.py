"""Parity of the HIP path with the CPU oracle, through the C ABI, on the GPU.

Paths: every token, bit-exact except counted near-ties; a flipped token's
device path is re-evaluated by the oracle and every decision on it must
follow its logit's sign.  y: every token, at every size (flipped tokens
against the oracle along the device's paths); tolerance 1e-4 for fp32 and
2e-2 for bf16 (max elementwise relative error with the denominator floored
at the row RMS).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads
import sparse_tree_structured_amd as fff
from gpu_helpers import check, run, to_device, to_f64

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


@functools.lru_cache(maxsize=None)
def wl(name):
    return workloads.workload(name)


ALL = ["tiny", "gpt125m", "opt1p3b_d4", "opt1p3b_d6", "decode_skew_t1", "decode_skew_t8",
       "decode_skew_t64"]


@needs_gpu
@pytest.mark.parametrize("name", ALL)
def test_workload_default_plan(name):
    inp = wl(name)
    y, path = run(inp)
    r = check(inp, y, path)
    print(name, r)


@needs_gpu
@pytest.mark.parametrize("name", ["tiny", "gpt125m", "decode_skew_t64"])
def test_workload_generic(name):
    inp = wl(name)
    y, path = run(inp, algo="generic")
    check(inp, y, path)


SHAPES = [
    # T, d, P, D, h, dtype
    (1, 64, 1, 0, 64, "bf16"),
    (1000, 128, 3, 4, 64, "bf16"),     # ragged T
    (333, 192, 2, 7, 128, "bf16"),
    (77, 64, 4, 10, 64, "bf16"),       # deep trees
    (50, 37, 3, 3, 5, "bf16"),         # odd widths -> generic
    (50, 37, 3, 3, 5, "f32"),
    (129, 96, 5, 2, 24, "f32"),
    (1, 1, 1, 0, 1, "f32"),
    (257, 256, 2, 6, 64, "bf16"),
    (100, 128, 2, 3, 512, "bf16"),     # wide nodes: H built by a separate pass
    (300, 512, 40, 2, 64, "bf16"),     # trees that do not fill the last tile
]


@needs_gpu
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_shape_sweep(shape):
    T, d, P, D, h, dt = shape
    inp = workloads.random_inputs(T, d, P, D, h, dt, seed=3, unit_rms_x=True)
    y, path = run(inp)
    check(inp, y, path)


@needs_gpu
@pytest.mark.parametrize("T,P", [(16420, 32), (32640, 32), (16420, 30)])
def test_split_top_levels(T, P):
    # Depth 6 takes the token-tile plan (k = 3); with one 256-column tile of
    # top-level columns and 129 or 255 token tiles of 128, the dense levels
    # run as two K halves that the token-tile kernel sums and walks.  T =
    # 16420 leaves 36 tokens in the last tile; P = 30 leaves the last group
    # of four trees two short.
    inp = workloads.random_inputs(T, 256, P, 6, 64, "bf16", seed=5, unit_rms_x=True)
    y, path = run(inp)
    check(inp, y, path)


@needs_gpu
def test_zero_weights_route_right():
    inp = workloads.random_inputs(100, 128, 2, 5, 64, "bf16", seed=1)
    inp.W_node[:] = 0
    inp.b_node[:] = 0
    y, path = run(inp)
    assert (path == (1 << 5) - 1).all()
    assert (y == 0).all()


@needs_gpu
def test_hand_built_routing():
    # w_n = s_p * e_level(n), x in {+-1}: leaf bits are [s_p x_l > 0].
    D, P, T, d, h = 5, 2, 256, 64, 64
    inp = workloads.random_inputs(T, d, P, D, h, "bf16", seed=2)
    N = (1 << (D + 1)) - 1
    rng = np.random.default_rng(0)
    xs = rng.choice([-1.0, 1.0], size=(T, D + 1))
    x = np.zeros((T, d))
    x[:, :D + 1] = xs
    W = np.zeros((P, N, d))
    s = np.array([1.0, -1.0])
    for n in range(N):
        W[:, n, int(np.log2(n + 1))] = s
    inp.x[:] = workloads.round_to_bf16_bits(x)
    inp.W_node[:] = workloads.round_to_bf16_bits(W)
    inp.b_node[:] = 0
    y, path = run(inp)
    for p in range(P):
        leaf = np.zeros(T, dtype=np.int64)
        for lvl in range(D):
            leaf |= (s[p] * xs[:, lvl] > 0).astype(np.int64) << (D - 1 - lvl)
        np.testing.assert_array_equal(path[:, p], leaf)
    check(inp, y, path)


@needs_gpu
def test_deterministic():
    inp = wl("gpt125m")
    y1, p1 = run(inp)
    y2, p2 = run(inp)
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(y1, y2)


@needs_gpu
def test_batch_invariance_decode():
    paths = {}
    for T in (1, 8, 64):
        _, paths[T] = run(wl(f"decode_skew_t{T}"))
    np.testing.assert_array_equal(paths[8], paths[64][:8])
    np.testing.assert_array_equal(paths[1], paths[64][:1])


@needs_gpu
def test_empty_leaves_in_skewed_workload():
    _, path = run(wl("decode_skew_t64"))
    used = np.zeros((path.shape[1], 64), dtype=bool)
    for p in range(path.shape[1]):
        used[p, path[:, p]] = True
    empty = 1.0 - used.mean()
    assert empty > 0.3, empty  # the raised biases starve whole subtrees


@needs_gpu
def test_zero_tokens():
    import sparse_tree_structured_amd as fff
    inp = workloads.random_inputs(0, 64, 2, 3, 64, "bf16")
    T = to_device(inp)
    y, path = fff.forward(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"])
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and path.shape == (0, 2)


@needs_gpu
@pytest.mark.parametrize("M,K,N", [(16384, 4096, 2048), (1000, 1024, 768), (1, 64, 8), (129, 192, 72),
                                   # direct-to-LDS with 128 x 128 tiles: a ragged last
                                   # column tile of 8 columns, and ragged rows
                                   (8192, 1024, 776), (4000, 4096, 2048)])
def test_projection_matches_fp64(M, K, N):
    import sparse_tree_structured_amd as fff
    g = torch.Generator().manual_seed(M + K + N)
    H = torch.randn(M, K, generator=g).to(torch.bfloat16)
    Wo = (torch.randn(K, N, generator=g) / K ** 0.5).to(torch.bfloat16)
    ref = H.double() @ Wo.double()  # every row, in float64 on the CPU
    for algo in ("prefill", "generic"):
        if algo == "prefill" and K % 64:
            continue
        for use_ws in (True, False):  # fff_project_ws and fff_project
            y = fff.project(H.cuda(), Wo.cuda(), algo=algo, use_workspace=use_ws)
            torch.cuda.synchronize()
            got = to_f64(y)
            err = np.abs(got - ref.numpy()) / np.maximum(np.abs(ref.numpy()), 1e-2)
            assert err.max() < 2e-2, (algo, use_ws, err.max())


SPLITS = [
    # workload, split level k, chunk tokens (0 = auto)
    ("opt1p3b_d6", 3, 0),
    ("opt1p3b_d6", 7, 0),      # every level dense
    ("opt1p3b_d6", 4, 0),
    ("opt1p3b_d6", 3, 1000),   # chunks that do not divide T
    ("opt1p3b_d6", 3, 4096),   # bucketed (an explicit chunk) beside the token-tile path (chunk 0)
    ("opt1p3b_d4", 1, 0),
    ("opt1p3b_d4", 5, 0),
    ("gpt125m", 2, 0),
    ("gpt125m", 3, 256),
    ("gpt125m", 3, 3000),      # bucketing slices of 1000 tokens; last chunk 2192 tokens
    ("gpt125m", 6, 0),
    ("decode_skew_t64", 3, 16),
    ("decode_skew_t8", 6, 0),
]


@needs_gpu
@pytest.mark.parametrize("name,k,chunk", SPLITS, ids=[f"{n}-k{k}-c{c}" for n, k, c in SPLITS])
def test_prefill_split_levels(name, k, chunk):
    import sparse_tree_structured_amd as fff
    inp = wl(name)
    T = to_device(inp)
    print(f"[gpu] {name} k={k} chunk={chunk}", flush=True)
    y, path = fff.forward(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"],
                          algo="prefill", split_level=k, chunk_tokens=chunk)
    torch.cuda.synchronize()
    print(name, k, chunk, check(inp, to_f64(y), path.cpu().numpy()))


@needs_gpu
@pytest.mark.parametrize("name", ["gpt125m", "opt1p3b_d6"])
def test_route_matches_forward_h(name):
    # fff_route exposes H; projecting it must give fff_forward's y exactly
    # (at the OPT-1.3B shape through the direct-to-LDS product).
    import sparse_tree_structured_amd as fff
    inp = wl(name)
    T = to_device(inp)
    H, path = fff.route(T["x"], T["W_node"], T["b_node"], T["V_node"])
    y2 = fff.project(H, T["W_out"])
    y, path1 = fff.forward(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"])
    torch.cuda.synchronize()
    assert torch.equal(path, path1)
    assert torch.equal(y, y2)


DECODE_SHAPES = [
    # T, d, P, D, h (bf16)
    (1, 256, 2, 0, 256),       # a single level
    (5, 256, 4, 3, 128),       # ragged T
    (17, 512, 8, 5, 64),       # a last routing item holding one token
    (64, 2048, 32, 6, 128),    # unskewed: later rounds see up to 16 distinct nodes
    (33, 768, 4, 9, 128),      # three rounds
    (40, 256, 320, 3, 8),      # more routing items than workgroups
    (3, 256, 2, 15, 256),      # deepest tree and widest node output the kernel takes
    (64, 1024, 16, 7, 64),
    (8, 128, 4, 2, 128),       # narrowest model width
    (12, 256, 8, 4, 192),      # trees straddling K-chunk boundaries
    # T <= 8 and 4 <= D <= 7: one subtree item per level-(D-3) node
    (1, 128, 64, 4, 8),        # one top level, narrowest rows
    (6, 512, 8, 5, 64),        # two top levels, ragged T
    (8, 2048, 32, 6, 128),     # the decode workload's layer, unskewed
    (2, 1024, 16, 7, 64),      # four top levels: 256 items, the most that fit
    (8, 2048, 32, 7, 64),      # 512 items would not fit: round items instead
    (3, 256, 4, 6, 256),       # widest node output
    (7, 256, 24, 6, 64),       # eight trees per K chunk
    (4, 256, 8, 6, 192),       # trees straddling K-chunk boundaries
]


@needs_gpu
@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=[str(s) for s in DECODE_SHAPES])
def test_decode_shapes(shape):
    T, d, P, D, h = shape
    inp = workloads.random_inputs(T, d, P, D, h, "bf16", seed=5, unit_rms_x=True)
    y, path = run(inp, algo="decode")
    check(inp, y, path)


@needs_gpu
@pytest.mark.parametrize("name", ["decode_skew_t1", "decode_skew_t8", "decode_skew_t64"])
def test_decode_matches_prefill(name):
    inp = wl(name)
    yd, pd = run(inp, algo="decode")
    yp, pp = run(inp, algo="prefill")
    np.testing.assert_array_equal(pd, pp)
    # Same bf16 H on both paths; the projections differ only in fp32
    # summation order before the final rounding.
    assert np.abs(yd - yp).max() <= 2e-2 * np.sqrt(np.mean(yp ** 2))


@needs_gpu
def test_decode_workspace_reuse():
    # One workspace over calls of different sizes: the arrival counters are
    # reset inside each call; results repeat bit for bit.
    import sparse_tree_structured_amd as fff
    big = workloads.random_inputs(64, 512, 8, 4, 64, "bf16", seed=8, unit_rms_x=True)
    Tb = to_device(big)
    shape = fff.shape_of(Tb["x"], Tb["W_node"], Tb["V_node"])
    ws, _ = fff.alloc_workspace(shape, fff.make_plan("decode"), Tb["x"].device)
    outs = []
    for T in (64, 7, 64):
        x = Tb["x"][:T].contiguous()
        print(f"[gpu] decode reuse T={T}", flush=True)
        y, path = fff.forward(x, Tb["W_node"], Tb["b_node"], Tb["V_node"], Tb["W_out"],
                              algo="decode", workspace=ws)
        y2, _ = fff.forward(x, Tb["W_node"], Tb["b_node"], Tb["V_node"], Tb["W_out"],
                            algo="decode", want_path=False)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        outs.append((to_f64(y), path.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[2][0])
    np.testing.assert_array_equal(outs[0][1][:7], outs[1][1])
    check(big, outs[0][0], outs[0][1])


# Depth sweep (D = 0..11, the measurement beside a dense FF block): every
# depth on the path AUTO takes at the sweep's widths, at a ragged token count.
@needs_gpu
@pytest.mark.parametrize("D", list(range(12)))
def test_depth_sweep_depths(D):
    inp = workloads.random_inputs(300, 512, 8, D, 128, "bf16", seed=40 + D, unit_rms_x=True)
    y, path = run(inp)
    check(inp, y, path)


@needs_gpu
@pytest.mark.parametrize("D", [0, 8, 9])
def test_depth_sweep_full_width(D):
    # The sweep's own d, P and h (those of the OPT-1.3B-shaped workload).
    inp = workloads.random_inputs(200, 2048, 32, D, 128, "bf16", seed=60 + D, unit_rms_x=True)
    y, path = run(inp)
    check(inp, y, path)


@needs_gpu
@pytest.mark.parametrize("algo", ["generic", "prefill", "decode"])
def test_nan_logits_go_right(algo):
    # A NaN logit is not below zero, so it routes right on every path; the
    # affected trees' outputs (and y) are NaN on both sides.
    T = 8 if algo == "decode" else 300
    inp = workloads.random_inputs(T, 256, 8, 5, 64, "bf16", seed=13, unit_rms_x=True)
    nan_bf16 = np.uint16(0x7FC0)
    inp.b_node[:, [0, 2, 5]] = nan_bf16  # the root and two deeper nodes of every tree
    y, path = run(inp, algo=algo)
    f = inp.as_f64()
    ref = oracle.forward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"])
    np.testing.assert_array_equal(path, ref["path"])
    assert (path >= (1 << 4)).all()  # the root's decision was right for every token
    np.testing.assert_array_equal(np.isnan(y), np.isnan(ref["y"]))


@needs_gpu
def test_maximum_depth_generic():
    # D = 20 (the largest the boundary takes): 2^21 - 1 nodes per tree.
    inp = workloads.random_inputs(50, 8, 1, 20, 2, "f32", seed=14, unit_rms_x=True)
    y, path = run(inp)
    check(inp, y, path)


# The token-tile subtree kernel (split level k, chunk 0): every subtree
# count it instantiates (2^k for k = 1..5), 1 to 4 subtree levels, token
# counts that leave a ragged last tile, tree counts that leave a partial
# last tree group, and one token.
TILE = [
    # T, d, P, D, h, k
    (1000, 256, 5, 6, 128, 3),   # 512-token tiles, 4-tree groups: both ragged
    (300, 128, 3, 5, 64, 2),     # 256-token tiles of 8 trees
    (777, 256, 4, 4, 64, 1),     # 128-token tiles of 16 trees
    (600, 512, 2, 7, 128, 4),    # 16 subtrees per tree
    (513, 256, 3, 5, 64, 5),     # 32 subtrees of one level (the leaves)
    (400, 256, 6, 5, 128, 3),    # three-level subtrees
    (64, 2048, 32, 6, 128, 3),   # the decode workload's widths through the prefill path
    (1, 64, 1, 1, 64, 1),
    (2048, 2048, 32, 6, 128, 3),  # the headline widths, four full tiles
]


@needs_gpu
@pytest.mark.parametrize("shape", TILE, ids=[str(s) for s in TILE])
def test_subtree_tiles(shape):
    import sparse_tree_structured_amd as fff
    T, d, P, D, h, k = shape
    inp = workloads.random_inputs(T, d, P, D, h, "bf16", seed=90 + k, unit_rms_x=True)
    Td = to_device(inp)
    plan = fff.resolve_plan(fff.shape_of(Td["x"], Td["W_node"], Td["V_node"]),
                            fff.make_plan("prefill", k, 0))
    assert plan.split_level == k and plan.chunk_tokens == 0  # the token-tile path
    y, path = run(inp, algo="prefill", split_level=k)
    print(shape, check(inp, y, path))


@needs_gpu
@pytest.mark.parametrize("name,k", [("opt1p3b_d6", 3), ("gpt125m", 2), ("opt1p3b_d4", 1)])
def test_subtree_matches_dense_paths(name, k):
    # The token-tile path and the all-dense path take the same decisions
    # (bit for bit: the logits differ only in fp32 summation order, and no
    # decision of these workloads lies that close to zero); their y agree
    # to the bf16 tolerance (a rounding of H may land one bf16 step apart).
    from oracle.compare import y_error
    inp = wl(name)
    y1, p1 = run(inp, algo="prefill", split_level=k)
    y2, p2 = run(inp, algo="prefill", split_level=inp.shape.D + 1)
    np.testing.assert_array_equal(p1, p2)
    assert y_error(y1, y2)["err"] <= 2e-2


# Wide node outputs through the bucketed deep levels (v rows of 512 and
# 1024 bytes copied into LDS, h/32 columns per lane) and the dense H pass.
WIDE = [
    # T, d, P, D, h, split level (-1: AUTO)
    (300, 256, 3, 7, 256, 4),
    (200, 512, 2, 5, 512, 2),
    (300, 128, 4, 3, 256, -1),
]


@needs_gpu
@pytest.mark.parametrize("shape", WIDE, ids=[str(s) for s in WIDE])
def test_wide_nodes(shape):
    T, d, P, D, h, k = shape
    inp = workloads.random_inputs(T, d, P, D, h, "bf16", seed=61 + D, unit_rms_x=True)
    y, path = run(inp, algo="prefill", split_level=k)
    check(inp, y, path)
