"""The C-ABI library on the CPU: it loads, exports what include/fff.h
declares, and its host-side validation returns the documented codes before
any HIP call (only error paths and T=0 are exercised here; no kernel runs)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_tree_structured_amd as fff

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fff.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fff.LIBRARY):
        from sparse_tree_structured_amd import build
        build.build()
    return fff.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fff_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fff.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(5):
        assert fff.status_string(code)
    assert fff.status_string(99) == "unknown status"
    assert [fff.algo_name(a) for a in range(4)] == ["auto", "generic", "prefill", "decode"]


def _shape(**kw):
    base = dict(T=64, d=64, P=2, D=3, h=32, dtype=fff.DTYPE_BF16)
    base.update(kw)
    return fff.make_shape(**base)


FAKE = 0x10000  # an aligned, never-dereferenced address: validation fails first


def _forward(lib, shape, plan=None, ptrs=None, path=FAKE, ws=FAKE, ws_bytes=1 << 40):
    p = dict(x=FAKE, W=FAKE, b=FAKE, V=FAKE, Wo=FAKE, y=FAKE)
    p.update(ptrs or {})
    return lib.fff_forward(ctypes.byref(shape), ctypes.byref(plan) if plan else None, p["x"], p["W"],
                           p["b"], p["V"], p["Wo"], p["y"], path, ws, ws_bytes, None, None)


@pytest.mark.parametrize("kw", [dict(T=-1), dict(d=0), dict(P=0), dict(h=0), dict(D=-1),
                                dict(D=fff.MAX_DEPTH + 1), dict(T=1 << 31), dict(d=(1 << 22) + 1),
                                dict(T=1 << 30, P=4)])
def test_bad_shapes(lib, kw):
    assert _forward(lib, _shape(**kw)) == fff.ERROR_INVALID_VALUE
    n = ctypes.c_size_t()
    assert lib.fff_workspace_size(ctypes.byref(_shape(**kw)), None, ctypes.byref(n)) == \
        fff.ERROR_INVALID_VALUE


@pytest.mark.parametrize("variant", [-1, 2, 1 << 20])
def test_bad_variant(lib, variant):
    assert _forward(lib, _shape(variant=variant)) == fff.ERROR_INVALID_VALUE
    n = ctypes.c_size_t()
    assert lib.fff_workspace_size(ctypes.byref(_shape(variant=variant)), None,
                                  ctypes.byref(n)) == fff.ERROR_INVALID_VALUE


def test_variant_does_not_change_plans(lib):
    # FFF-post moves the GELU only: every shape gets the same plan and workspace.
    for kw in (dict(), dict(dtype=fff.DTYPE_F32), dict(T=8, d=2048, P=32, D=6, h=128),
               dict(T=16384, d=2048, P=32, D=6, h=128), dict(T=500, d=256, P=4, D=10, h=64)):
        a, b = _shape(**kw), _shape(variant=fff.VARIANT_POST, **kw)
        pa, pb = fff.plan_default(a), fff.plan_default(b)
        assert (pa.algo, pa.split_level, pa.chunk_tokens) == (pb.algo, pb.split_level,
                                                              pb.chunk_tokens)
        assert fff.workspace_size(a) == fff.workspace_size(b)
    assert fff.make_shape(1, 1, 1, 0, 1, fff.DTYPE_F32, "post").variant == fff.VARIANT_POST


def test_unknown_dtype(lib):
    assert _forward(lib, _shape(dtype=7)) == fff.ERROR_NOT_SUPPORTED


def test_null_shape_and_outputs(lib):
    n = ctypes.c_size_t()
    assert lib.fff_workspace_size(None, None, ctypes.byref(n)) == fff.ERROR_INVALID_VALUE
    assert lib.fff_workspace_size(ctypes.byref(_shape()), None, None) == fff.ERROR_INVALID_VALUE
    assert lib.fff_plan_default(ctypes.byref(_shape()), None) == fff.ERROR_INVALID_VALUE


@pytest.mark.parametrize("which", ["x", "W", "b", "V", "Wo", "y"])
def test_null_pointers(lib, which):
    assert _forward(lib, _shape(), ptrs={which: None}) == fff.ERROR_INVALID_VALUE


@pytest.mark.parametrize("which", ["x", "W", "V", "Wo", "y"])
def test_misaligned_pointers(lib, which):
    assert _forward(lib, _shape(), ptrs={which: FAKE + 2}) == fff.ERROR_INVALID_VALUE


def test_misaligned_bias_and_path(lib):
    assert _forward(lib, _shape(dtype=fff.DTYPE_F32), ptrs={"b": FAKE + 2}) == fff.ERROR_INVALID_VALUE
    assert _forward(lib, _shape(), path=FAKE + 2) == fff.ERROR_INVALID_VALUE


def test_workspace_checks(lib):
    s = _shape()
    need = fff.workspace_size(s)
    assert need > 0
    assert _forward(lib, s, ws_bytes=need - 1) == fff.ERROR_WORKSPACE
    assert _forward(lib, s, ws=None) == fff.ERROR_WORKSPACE
    assert _forward(lib, s, ws=FAKE + 16) == fff.ERROR_INVALID_VALUE


def test_zero_tokens_is_a_noop(lib):
    s = _shape(T=0)
    assert fff.workspace_size(s) == 0
    nulls = dict(x=None, W=None, b=None, V=None, Wo=None, y=None)
    assert _forward(lib, s, ptrs=nulls, path=None, ws=None, ws_bytes=0) == fff.SUCCESS
    assert lib.fff_project(ctypes.byref(s), fff.ALGO_AUTO, None, None, None, None) == fff.SUCCESS


def test_plans(lib):
    p = fff.plan_default(_shape(dtype=fff.DTYPE_F32))
    assert p.algo == fff.ALGO_GENERIC
    p = fff.plan_default(_shape(T=16384, d=2048, P=32, D=6, h=128))
    assert p.algo in (fff.ALGO_PREFILL, fff.ALGO_DECODE)
    # PREFILL needs bf16 and 64-aligned widths.
    bad = fff.make_plan(fff.ALGO_PREFILL)
    assert _forward(lib, _shape(dtype=fff.DTYPE_F32), plan=bad) == fff.ERROR_NOT_SUPPORTED
    assert _forward(lib, _shape(d=72), plan=bad) == fff.ERROR_NOT_SUPPORTED
    assert _forward(lib, _shape(), plan=fff.make_plan(9)) == fff.ERROR_INVALID_VALUE
    # Plan flags: the defined bit passes through resolution; others are invalid.
    dec = _shape(T=8, d=2048, P=32, D=6, h=128)
    r = fff.resolve_plan(dec, fff.make_plan("decode", flags=fff.PLAN_TEST_DECODE_NO_PUBLISH))
    assert r.algo == fff.ALGO_DECODE and r.flags == fff.PLAN_TEST_DECODE_NO_PUBLISH
    assert fff.resolve_plan(dec, fff.make_plan()).flags == 0
    for flags in (2, 1 << 30, -1):
        assert _forward(lib, dec, plan=fff.make_plan(flags=flags)) == fff.ERROR_INVALID_VALUE
        assert lib.fff_plan_resolve(ctypes.byref(dec), ctypes.byref(fff.make_plan(flags=flags)),
                                    ctypes.byref(fff.Plan())) == fff.ERROR_INVALID_VALUE


def test_deep_chunk_rule():
    # Bucketed deep levels: about 32 MB of x rows per chunk, at least 64
    # tokens per level-k bucket on average, at most T.
    wide = dict(T=16384, d=2048, P=32, h=128)
    for D, k, chunk in ((8, 5, 8192), (9, 6, 8192), (10, 7, 8192), (11, 8, 16384)):
        r = fff.resolve_plan(_shape(D=D, **wide), fff.make_plan("prefill"))
        assert (r.split_level, r.chunk_tokens) == (k, chunk), (D, r.split_level, r.chunk_tokens)
    r = fff.resolve_plan(_shape(T=300, d=512, P=8, D=11, h=128), fff.make_plan("prefill"))
    assert (r.split_level, r.chunk_tokens) == (8, 300)
    r = fff.resolve_plan(_shape(T=100000, d=512, P=8, D=9, h=128), fff.make_plan("prefill"))
    assert r.chunk_tokens == 32768  # 32 MB of 1 KB rows


def test_project_validation(lib):
    s = _shape()
    assert lib.fff_project(ctypes.byref(s), 7, FAKE, FAKE, FAKE, None) == fff.ERROR_INVALID_VALUE
    assert lib.fff_project(ctypes.byref(s), fff.ALGO_AUTO, None, FAKE, FAKE, None) == \
        fff.ERROR_INVALID_VALUE
    assert lib.fff_project(ctypes.byref(_shape(dtype=fff.DTYPE_F32)), fff.ALGO_PREFILL, FAKE, FAKE,
                           FAKE, None) == fff.ERROR_NOT_SUPPORTED


def test_decode_plans(lib):
    dec = dict(d=2048, P=32, D=6, h=128)
    for T in (1, 8, 64):
        assert fff.plan_default(_shape(T=T, **dec)).algo == fff.ALGO_DECODE
    # More than 64 tokens, fp32, or widths the kernel does not take: staged.
    assert fff.plan_default(_shape(T=65, **dec)).algo == fff.ALGO_PREFILL
    assert fff.plan_default(_shape(T=8, **dict(dec, d=2304))).algo == fff.ALGO_PREFILL
    assert fff.plan_default(_shape(T=8, **dict(dec, h=120))).algo == fff.ALGO_GENERIC
    assert fff.plan_default(_shape(T=8, dtype=fff.DTYPE_F32, **dec)).algo == fff.ALGO_GENERIC
    forced = fff.make_plan("decode")
    for kw in (dict(T=65), dict(T=8, d=192), dict(T=8, d=2176), dict(T=8, D=16), dict(T=8, h=512),
               dict(T=8, P=3, h=128), dict(T=8, dtype=fff.DTYPE_F32)):
        s = _shape(**dict(dec, **kw))
        assert _forward(lib, s, plan=forced) == fff.ERROR_NOT_SUPPORTED, kw
    r = fff.resolve_plan(_shape(T=8, **dec), forced)
    assert r.algo == fff.ALGO_DECODE and r.split_level == 0 and r.chunk_tokens == 0


def test_decode_workspace_covers_route(lib):
    # fff_route never runs the fused kernel: AUTO resolves to a staged
    # algorithm there, and the size reported for AUTO covers both.
    s = _shape(T=8, d=2048, P=32, D=6, h=128)
    auto = fff.workspace_size(s)
    dec = fff.workspace_size(s, fff.make_plan("decode"))
    pre = fff.workspace_size(s, fff.make_plan("prefill"))
    assert auto >= dec > 0 and auto >= pre > 0
    # A 256-byte epoch header, 128 routing-item slots (2 tokens per item at
    # 8 tokens; 64-bit each), H [8, 4096] bf16, 32 x 8 arrival slots and 8
    # K-chunk partials of y [8, 2048] fp32.
    assert dec == 256 + 32 * 4 * 8 + 8 * 4096 * 2 + 32 * 8 * 8 + 8 * 8 * 2048 * 4
    # 9 tokens: 2 tokens per item, 5 items per tree.
    s9 = _shape(T=9, d=2048, P=32, D=6, h=128)
    assert fff.workspace_size(s9, fff.make_plan("decode")) == \
        256 + 32 * 5 * 8 + 9 * 4096 * 2 + 32 * 8 * 8 + 8 * 9 * 2048 * 4
    # 64 tokens: 8 per item, 8 items per tree (256 items fit half of the grid).
    s64 = _shape(T=64, d=2048, P=32, D=6, h=128)
    assert fff.workspace_size(s64, fff.make_plan("decode")) == \
        256 + 32 * 8 * 8 + 64 * 4096 * 2 + 32 * 8 * 8 + 8 * 64 * 2048 * 4
    # 64 tokens on 64 trees: 16 per item (8-token items would be 512).
    w64 = _shape(T=64, d=2048, P=64, D=6, h=128)
    assert fff.workspace_size(w64, fff.make_plan("decode")) == \
        256 + 64 * 4 * 8 + 64 * 8192 * 2 + 32 * 16 * 8 + 16 * 64 * 2048 * 4
    st = lib.fff_route(ctypes.byref(s), ctypes.byref(fff.make_plan("decode")), FAKE, FAKE, FAKE,
                       FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == fff.ERROR_NOT_SUPPORTED


def test_prune_table_size():
    # Alive flags [P][N]; for PREFILL also the packed rows of the dense
    # levels (at most P tiles of 256 columns) and their maps.
    dec = _shape(T=8, d=2048, P=32, D=6, h=128)
    assert fff.prune_table_size(dec) == 4096  # 32 * 127 bytes, rounded to 256
    pre = _shape(T=16384, d=2048, P=32, D=6, h=128)
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    # alive flags, tree bases, tile first/count, column map and info, packed rows
    expect = up(32 * 127) + 3 * up(32 * 4) + 2 * up(32 * 256 * 4) + up(32 * 256 * 2048 * 2)
    assert fff.prune_table_size(pre) == expect
    split = fff.resolve_plan(pre, fff.make_plan("prefill", 4))
    assert split.split_level == 4
    assert fff.prune_table_size(pre, split) == expect  # bounded by P tiles either way


def _prepare(lib, shape, mask, W=FAKE, table=FAKE, nbytes=1 << 40, out=True):
    res = fff.Pruning()
    m = np.ascontiguousarray(mask, dtype=np.uint8) if mask is not None else None
    return lib.fff_prune_prepare(ctypes.byref(shape), None,
                                 m.ctypes.data_as(ctypes.c_void_p) if m is not None else None, W,
                                 table, nbytes, None, ctypes.byref(res) if out else None)


def test_prune_prepare_validation(lib):
    s = _shape(T=1000, d=128, P=3, D=4, h=64)
    mask = np.ones((3, 16), np.uint8)
    dead = mask.copy()
    dead[1] = 0  # a tree with no alive leaf
    assert _prepare(lib, s, dead) == fff.ERROR_INVALID_VALUE
    assert _prepare(lib, s, None) == fff.ERROR_INVALID_VALUE
    assert _prepare(lib, s, mask, W=None) == fff.ERROR_INVALID_VALUE
    assert _prepare(lib, s, mask, table=None) == fff.ERROR_INVALID_VALUE
    assert _prepare(lib, s, mask, table=FAKE + 16) == fff.ERROR_INVALID_VALUE
    assert _prepare(lib, s, mask, out=False) == fff.ERROR_INVALID_VALUE
    assert _prepare(lib, s, mask, nbytes=fff.prune_table_size(s) - 1) == fff.ERROR_WORKSPACE


def test_forward_pruned_validation(lib):
    s = _shape(T=1000, d=128, P=3, D=4, h=64)
    plan = fff.resolve_plan(s, fff.make_plan("auto"))
    assert plan.algo == fff.ALGO_PREFILL and plan.split_level == 5

    def run(pr, pl=None):
        return lib.fff_forward_pruned(ctypes.byref(s), ctypes.byref(pl) if pl else None,
                                      ctypes.byref(pr) if pr is not None else None, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None, None)

    good = dict(table=FAKE, P=3, D=4, d=128, split_level=5, col_tiles=1)
    assert run(None) == fff.ERROR_INVALID_VALUE
    for bad in (dict(table=None), dict(table=FAKE + 8), dict(P=4), dict(D=3), dict(d=64),
                dict(split_level=9), dict(col_tiles=4), dict(col_tiles=0)):
        assert run(fff.Pruning(**dict(good, **bad))) == fff.ERROR_INVALID_VALUE, bad
    # A PREFILL plan must use the split level the table packed.
    assert run(fff.Pruning(**dict(good, split_level=3))) == fff.ERROR_NOT_SUPPORTED
    assert run(fff.Pruning(**good), fff.make_plan("prefill", 3)) == fff.ERROR_NOT_SUPPORTED


def test_backward_plans_and_workspace():
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    # AUTO takes the matrix-core path where every level is dense.
    s = _shape(T=16384, d=2048, P=32, D=6, h=128)
    assert fff.backward_workspace_size(s) == fff.backward_workspace_size(s, fff.make_plan("prefill"))
    T, Tp, cols, K, d = 16384, 16384, 32 * 128, 32 * 128, 2048
    expect = (up(T * 32 * 7 * 4) + up(T * 32 * 4) + 2 * up(d * Tp * 2) + up(K * Tp * 4) +
              up(T * cols * 2) + 2 * up(cols * Tp * 2) + 2 * up(K * Tp * 2) + up(d * cols * 2) +
              up(max(2 * 32 * 127 * d, 2 * K * d, 8 * 32 * 127 * 128) * 4))  # split partials
    assert fff.backward_workspace_size(s) == expect
    # Generic for fp32, deep (split) trees and shallow trees.
    g = _shape(T=100, d=64, P=2, D=3, h=32, dtype=fff.DTYPE_F32)
    assert fff.backward_workspace_size(g) == up(100 * 2 * 4 * 4) + up(100 * 2 * 4) + \
        2 * up(100 * 64 * 4) + up(100 * 64 * 4)
    for shp in (_shape(T=100, d=2048, P=32, D=8, h=128), _shape(T=100, d=64, P=2, D=1, h=64)):
        with pytest.raises(fff.FFFError):
            fff.backward_workspace_size(shp, fff.make_plan("prefill"))
    with pytest.raises(fff.FFFError):
        fff.backward_workspace_size(s, fff.make_plan("decode"))
    with pytest.raises(fff.FFFError):
        fff.backward_workspace_size(s, fff.make_plan("prefill", 4))


def test_backward_pruned_plans_and_validation(lib):
    s = _shape(T=16384, d=2048, P=32, D=6, h=128)
    dense = dict(table=FAKE, P=32, D=6, d=2048, split_level=7, col_tiles=16)
    tile = dict(dense, split_level=3, col_tiles=1)
    # A table with every level packed: AUTO takes the matrix-core backward,
    # whose workspace is the unpruned one's.
    full = fff.backward_workspace_size(s)
    assert fff.backward_pruned_workspace_size(s, None, fff.Pruning(**dense)) == full
    assert fff.backward_pruned_workspace_size(s, fff.make_plan("prefill"),
                                              fff.Pruning(**dense)) == full
    # Any other table: AUTO takes the generic backward; PREFILL is refused.
    generic = fff.backward_workspace_size(s, fff.make_plan("generic"))
    assert generic != full
    assert fff.backward_pruned_workspace_size(s, None, fff.Pruning(**tile)) == generic
    with pytest.raises(fff.FFFError) as err:
        fff.backward_pruned_workspace_size(s, fff.make_plan("prefill"), fff.Pruning(**tile))
    assert err.value.status == fff.ERROR_NOT_SUPPORTED

    def run(pr, pl=None, nbytes=1 << 40, ws=FAKE, outs=FAKE):
        return lib.fff_backward_pruned(
            ctypes.byref(s), ctypes.byref(pl) if pl else None,
            ctypes.byref(pr) if pr is not None else None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, outs, outs, outs, outs, ws, nbytes, None)

    assert run(None) == fff.ERROR_INVALID_VALUE
    for bad in (dict(table=None), dict(table=FAKE + 8), dict(P=4), dict(D=5), dict(d=64),
                dict(split_level=9), dict(col_tiles=33), dict(col_tiles=0)):
        assert run(fff.Pruning(**dict(dense, **bad))) == fff.ERROR_INVALID_VALUE, bad
        assert lib.fff_backward_pruned_workspace_size(
            ctypes.byref(s), None, ctypes.byref(fff.Pruning(**dict(dense, **bad))),
            ctypes.byref(ctypes.c_size_t())) == fff.ERROR_INVALID_VALUE, bad
    assert run(fff.Pruning(**tile), fff.make_plan("prefill")) == fff.ERROR_NOT_SUPPORTED
    assert run(fff.Pruning(**dense), fff.make_plan("decode")) == fff.ERROR_NOT_SUPPORTED
    assert run(fff.Pruning(**dense), outs=None) == fff.ERROR_INVALID_VALUE
    assert run(fff.Pruning(**dense), nbytes=full - 1) == fff.ERROR_WORKSPACE
    assert run(fff.Pruning(**dense), ws=FAKE + 16) == fff.ERROR_INVALID_VALUE


@pytest.mark.parametrize("D,k,chunk,slices", [(8, 5, 8192, 8), (11, 8, 16384, 16)])
def test_bucketed_plan_workspace(D, k, chunk, slices):
    # Bucketed plans carve per-(chunk, tree) offsets and per-(chunk, tree,
    # slice) counts; the slices per chunk aim at about 512 workgroups of
    # 1024 tokens at most each, at most 16.
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    T, d, P, h = 16384, 2048, 32, 128
    s = _shape(T=T, d=d, P=P, D=D, h=h)
    plan = fff.resolve_plan(s, fff.make_plan())
    assert (plan.algo, plan.split_level, plan.chunk_tokens) == (fff.ALGO_PREFILL, k, chunk)
    nch = T // chunk
    expect = (up(T * P * k * 4) + up(T * P * 4) + up(T * P * 4) + up(nch * P * (2 ** k + 1) * 4)
              + up(nch * P * slices * 2 ** k * 4) + up(T * P * h * 2))  # W_out used as it is
    assert fff.workspace_size(s) == expect


def test_project_ws_sizes_and_validation(lib):
    n = ctypes.c_size_t()
    big = fff.make_shape(16384, 2048, 1, 0, 4096, fff.DTYPE_BF16)   # y = H[16384,4096] . W[4096,2048]
    # No projection kernel needs workspace (the direct-to-LDS product reads
    # W_out in its own layout).
    assert fff.project_workspace_size(big) == 0
    assert fff.project_workspace_size(big, "prefill") == 0
    assert fff.project_workspace_size(big, "generic") == 0
    small = fff.make_shape(1000, 768, 1, 0, 1024, fff.DTYPE_BF16)  # too few output tiles
    assert fff.project_workspace_size(small) == 0
    f32 = fff.make_shape(16384, 2048, 1, 0, 4096, fff.DTYPE_F32)
    assert fff.project_workspace_size(f32) == 0
    assert lib.fff_project_workspace_size(ctypes.byref(big), 7, ctypes.byref(n)) == \
        fff.ERROR_INVALID_VALUE
    assert lib.fff_project_workspace_size(ctypes.byref(big), fff.ALGO_AUTO, None) == \
        fff.ERROR_INVALID_VALUE
    # All of these fail validation before any HIP call.
    ws = lib.fff_project_ws
    assert ws(ctypes.byref(big), 7, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == fff.ERROR_INVALID_VALUE
    assert ws(ctypes.byref(big), fff.ALGO_AUTO, None, FAKE, FAKE, FAKE, 1 << 30, None) == \
        fff.ERROR_INVALID_VALUE
    assert ws(ctypes.byref(f32), fff.ALGO_PREFILL, FAKE, FAKE, FAKE, None, 0, None) == \
        fff.ERROR_NOT_SUPPORTED
    assert ws(ctypes.byref(big), fff.ALGO_AUTO, FAKE, FAKE + 8, FAKE, None, 0, None) == \
        fff.ERROR_INVALID_VALUE  # W_out not 16-byte aligned
    empty = fff.make_shape(0, 2048, 1, 0, 4096, fff.DTYPE_BF16)
    assert ws(ctypes.byref(empty), fff.ALGO_AUTO, None, None, None, None, 0, None) == fff.SUCCESS


def test_static_forward_validation(lib):
    # fff_forward_static: validation, and a workspace beyond the fixed region,
    # return before any HIP call (FAKE pointers are never touched).
    def call(shape, plan=None):
        return lib.fff_forward_static(ctypes.byref(shape), ctypes.byref(plan) if plan else None,
                                      FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert call(_shape(T=-1)) == fff.ERROR_INVALID_VALUE
    assert call(_shape(dtype=7)) == fff.ERROR_NOT_SUPPORTED
    big = _shape(T=65536, d=64, P=4, D=3, h=128)
    n = ctypes.c_size_t()
    assert lib.fff_workspace_size(ctypes.byref(big), None, ctypes.byref(n)) == fff.SUCCESS
    assert n.value > fff.STATIC_SCRATCH_BYTES
    assert call(big) == fff.ERROR_WORKSPACE
    assert call(_shape(T=0)) == fff.SUCCESS


def test_token_tile_plans():
    # Split plans with chunk 0 take the token-tile subtree kernel where it
    # applies (1 <= k <= 5, at most four levels below k, every level's
    # records feeding the H pass: D + 1 <= 8); the resolved chunk stays 0 and
    # the workspace holds all D + 1 logits per (tree, token).  An explicit
    # chunk keeps the bucketed kernels.
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    T, d, P, h = 16384, 2048, 32, 128
    s = _shape(T=T, d=d, P=P, D=6, h=h)
    r = fff.resolve_plan(s, fff.make_plan("prefill", 3, 0))
    assert (r.split_level, r.chunk_tokens) == (3, 0)
    # ... plus, at this shape (one 256-column tile of top-level columns, 128
    # token tiles of 128), the two K halves of the dense levels' fp32 logits.
    expect = up(T * P * 7 * 4) + up(T * P * 4) + up(T * P * h * 2) + up(2 * 256 * T * 4)
    assert fff.workspace_size(s, r) == expect
    # Half the tokens: 64 token tiles, two halves still under 256 workgroups,
    # so the dense levels keep their own walk and no halves are stored.
    s2 = _shape(T=T // 2, d=d, P=P, D=6, h=h)
    r2 = fff.resolve_plan(s2, fff.make_plan("prefill", 3, 0))
    assert fff.workspace_size(s2, r2) == (up(T // 2 * P * 7 * 4) + up(T // 2 * P * 4) +
                                          up(T // 2 * P * h * 2))
    r = fff.resolve_plan(s, fff.make_plan("prefill", 3, 4096))
    assert (r.split_level, r.chunk_tokens) == (3, 4096)
    # k = 6 > 5 at depth 6: bucketed
    r = fff.resolve_plan(s, fff.make_plan("prefill", 6, 0))
    assert r.chunk_tokens > 0
    # AUTO: depth 6 and 7 keep the last four levels for the token-tile kernel
    for D in (6, 7):
        r = fff.resolve_plan(_shape(T=T, d=d, P=P, D=D, h=h), fff.make_plan())
        assert (r.algo, r.split_level, r.chunk_tokens) == (fff.ALGO_PREFILL, D - 3, 0)
    # depths 4 and 5 stay dense
    for D in (4, 5):
        r = fff.resolve_plan(_shape(T=T, d=d, P=P, D=D, h=h), fff.make_plan())
        assert (r.algo, r.split_level) == (fff.ALGO_PREFILL, D + 1)
    # depth 8 needs the bucketed kernels (the H pass takes at most 8 levels)
    r = fff.resolve_plan(_shape(T=T, d=d, P=P, D=8, h=h), fff.make_plan("prefill", 5, 0))
    assert r.chunk_tokens > 0
