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


def random_leaf_mask(rng, P, D, frac):
    """A seeded fraction of each tree's leaves pruned; every tree keeps one."""
    m = (rng.random((P, 1 << D)) >= frac).astype(np.uint8)
    m[np.arange(P), rng.integers(0, 1 << D, size=P)] = 1
    return m


def run_backward_pruned(inp, mask, algo="auto", table_algo="generic", table_split=-1,
                        variant=0, seed=7):
    """fff_backward_pruned on a table prepared for (table_algo, table_split),
    and the paths fff_forward_pruned takes on it (generic plan)."""
    T = to_device(inp)
    s = inp.shape
    dy_t, dy64 = make_dy(inp, seed)
    dy_t = dy_t.to(T["x"].device)
    print(f"[gpu] backward pruned {s} algo={algo} table={table_algo}/{table_split} "
          f"alive={mask.mean():.2f} variant={variant}", flush=True)
    pr, table = fff.prune_prepare(mask, T["W_node"], T["V_node"], algo=table_algo,
                                  split_level=table_split, T=max(s.T, 65536), variant=variant)
    g = fff.backward_pruned(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"], dy_t, pr,
                            algo=algo, variant=variant)
    _, path = fff.forward_pruned(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"], pr,
                                 algo="generic", variant=variant)
    torch.cuda.synchronize()
    del table
    return {k: to_f64(v) for k, v in g.items()}, path.cpu().numpy(), dy64


def check_grads_pruned(inp, mask, g, path, dy64, variant=0):
    f = inp.as_f64()
    rec = oracle.forward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"],
                         want_y=False, want_records=True, variant=variant, leaf_alive=mask)
    np.testing.assert_array_equal(path, rec["path"])
    ref = oracle.backward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"], dy64,
                          variant=variant, leaf_alive=mask)
    # Nodes no token visits (every pruned node among them) get exactly 0.
    s = inp.shape
    visited = np.zeros((s.P, (1 << (s.D + 1)) - 1), bool)
    nodes = np.asarray(rec["rec_node"]).reshape(s.T, s.P, s.D + 1)
    for p in range(s.P):
        visited[p, np.unique(nodes[:, p, :])] = True
    assert (g["db_node"][~visited] == 0).all()
    assert (g["dW_node"][~visited] == 0).all()
    assert (g["dV_node"][~visited] == 0).all()
    return assert_grads(s.dtype, g, ref, f, dy64, rec, variant)


PRUNED_GENERIC = [
    # T, d, P, D, h, dtype, pruned fraction
    (50, 37, 3, 3, 5, "f32", 0.5),
    (129, 96, 5, 2, 24, "f32", 0.7),
    (40, 64, 4, 4, 16, "bf16", 0.6),
    (33, 128, 3, 6, 64, "bf16", 0.8),
]


@needs_gpu
@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("case", PRUNED_GENERIC, ids=[str(c) for c in PRUNED_GENERIC])
def test_backward_pruned_generic(case, variant):
    T, d, P, D, h, dt, frac = case
    inp = workloads.random_inputs(T, d, P, D, h, dt, seed=90 + D, unit_rms_x=True)
    mask = random_leaf_mask(np.random.default_rng(5 + D), P, D, frac)
    g, path, dy = run_backward_pruned(inp, mask, algo="generic", variant=variant)
    check_grads_pruned(inp, mask, g, path, dy, variant=variant)


PRUNED_MFMA = [
    # T, d, P, D, h, pruned fraction  (bf16, every level dense)
    (300, 256, 4, 6, 64, 0.5),
    (1000, 128, 8, 2, 64, 0.5),
    (500, 512, 2, 7, 64, 0.7),
    (257, 256, 16, 5, 128, 0.3),
    (700, 256, 8, 6, 128, 0.9),   # a few paths left, packed into fewer column tiles
]


@needs_gpu
@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("case", PRUNED_MFMA, ids=[str(c) for c in PRUNED_MFMA])
def test_backward_pruned_mfma(case, variant):
    T, d, P, D, h, frac = case
    inp = workloads.random_inputs(T, d, P, D, h, "bf16", seed=110 + D, unit_rms_x=True)
    mask = random_leaf_mask(np.random.default_rng(9 + D), P, D, frac)
    g, path, dy = run_backward_pruned(inp, mask, algo="prefill", table_algo="prefill",
                                      table_split=D + 1, variant=variant)
    check_grads_pruned(inp, mask, g, path, dy, variant=variant)


@needs_gpu
def test_backward_pruned_token_tile_table():
    # A table prepared for the token-tile forward (split level 3 of 7) has
    # no packed rows for every level: AUTO takes the generic backward, and a
    # forced matrix-core plan is refused.
    inp = workloads.random_inputs(400, 256, 3, 6, 64, "bf16", seed=131, unit_rms_x=True)
    mask = random_leaf_mask(np.random.default_rng(13), 3, 6, 0.5)
    g, path, dy = run_backward_pruned(inp, mask, algo="auto", table_algo="prefill",
                                      table_split=3)
    check_grads_pruned(inp, mask, g, path, dy)
    T = to_device(inp)
    pr, table = fff.prune_prepare(mask, T["W_node"], T["V_node"], algo="prefill", split_level=3,
                                  T=65536)
    with pytest.raises(fff.FFFError) as err:
        fff.backward_pruned(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"],
                            T["x"].clone(), pr, algo="prefill")
    assert err.value.status == fff.ERROR_NOT_SUPPORTED
    del table


@needs_gpu
def test_backward_pruned_all_alive_equals_unpruned():
    # With every leaf alive the pruned backward is the unpruned one, bit for
    # bit on the matrix-core plan's deterministic gradients.
    inp = workloads.random_inputs(300, 256, 4, 6, 64, "bf16", seed=141, unit_rms_x=True)
    mask = np.ones((4, 64), np.uint8)
    g, _, _ = run_backward_pruned(inp, mask, algo="prefill", table_algo="prefill",
                                  table_split=7)
    g0, _, _ = run_backward(inp, algo="prefill")
    for k in ("dx", "dW_node", "dV_node", "dW_out"):
        np.testing.assert_array_equal(g[k], g0[k])


@needs_gpu
def test_backward_pruned_full_size_sampled():
    # The OPT-1.3B-shaped depth-6 layer with half of each tree's leaves
    # pruned, on the matrix-core plan, with dy nonzero on a sample of tokens
    # only (the oracle's pruned backward over the sample is then the exact
    # reference).
    inp = workloads.workload("opt1p3b_d6")
    s = inp.shape
    T = to_device(inp)
    mask = random_leaf_mask(np.random.default_rng(21), s.P, s.D, 0.5)
    print("[gpu] pruned backward full size", flush=True)
    pr, table = fff.prune_prepare(mask, T["W_node"], T["V_node"], algo="prefill",
                                  split_level=s.D + 1, T=s.T)
    _, path = fff.forward_pruned(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"], pr,
                                 algo="prefill", split_level=s.D + 1)
    torch.cuda.synchronize()
    path = path.cpu().numpy()
    cand = np.sort(np.random.default_rng(6).choice(s.T, size=48, replace=False))
    fc = inp.subset_tokens(cand).as_f64()
    ok = (oracle.forward(fc["x"], fc["W_node"], fc["b_node"], fc["V_node"], fc["W_out"],
                         want_y=False, leaf_alive=mask)["path"] == path[cand]).all(axis=1)
    rows = cand[ok][:24]
    assert len(rows) == 24
    dy = np.zeros((s.T, s.d))
    dy[rows] = np.random.default_rng(8).standard_normal((len(rows), s.d))
    dy_t = torch.from_numpy(dy).to(torch.bfloat16)
    dy64 = dy_t.double().numpy()
    g = fff.backward_pruned(T["x"], T["W_node"], T["b_node"], T["V_node"], T["W_out"],
                            dy_t.to(T["x"].device), pr)
    torch.cuda.synchronize()
    del table
    g = {k: to_f64(v) for k, v in g.items()}
    f = inp.subset_tokens(rows).as_f64()
    ref = oracle.backward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"], dy64[rows],
                          leaf_alive=mask)
    rec = oracle.forward(f["x"], f["W_node"], f["b_node"], f["V_node"], f["W_out"],
                         want_y=False, want_records=True, leaf_alive=mask)
    assert (g["dx"][np.setdiff1d(np.arange(s.T), rows)] == 0).all()
    g["dx"] = g["dx"][rows]
    assert_grads("bf16", g, ref, f, dy64[rows], rec, 0)
