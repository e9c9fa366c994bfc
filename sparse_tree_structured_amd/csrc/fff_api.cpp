// C ABI of the FFF forward pass: host-side validation, planning, workspace
// carving and kernel launches.  Validation runs before any HIP call, so every
// error path is testable without a GPU.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/fff.h"
#include "launch.hpp"

namespace {

using fff::Dims;

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr size_t kWsAlign = 256;
constexpr int32_t kPlanFlags = FFF_PLAN_TEST_DECODE_NO_PUBLISH;  // every defined plan flag

bool mul_ok(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

fff_status_t check_shape(const fff_shape_t* s, Dims* out) {
  if (!s) return FFF_ERROR_INVALID_VALUE;
  if (s->dtype != FFF_DTYPE_F32 && s->dtype != FFF_DTYPE_BF16) return FFF_ERROR_NOT_SUPPORTED;
  if (s->T < 0 || s->T > INT32_MAX || s->d <= 0 || s->P <= 0 || s->h <= 0 || s->D < 0 ||
      s->D > FFF_MAX_DEPTH || s->d > (1 << 22) ||
      (s->variant != FFF_VARIANT_FFF && s->variant != FFF_VARIANT_POST))
    return FFF_ERROR_INVALID_VALUE;
  Dims d;
  d.T = s->T;
  d.d = s->d;
  d.P = s->P;
  d.D = s->D;
  d.h = s->h;
  d.dtype = s->dtype;
  d.variant = s->variant;
  d.prune = nullptr;
  d.N = (int64_t(1) << (s->D + 1)) - 1;
  d.K = int64_t(s->P) * s->h;
  d.esize = s->dtype == FFF_DTYPE_F32 ? 4 : 2;
  // Every tensor must stay below 2^40 elements, and T*P below 2^31.
  if (!mul_ok(d.T, d.d, kMaxElems) || !mul_ok(int64_t(d.P) * d.N, d.d, kMaxElems) ||
      !mul_ok(int64_t(d.P) * d.N, d.h, kMaxElems) || !mul_ok(d.K, d.d, kMaxElems) ||
      !mul_ok(d.T, d.K, kMaxElems) || !mul_ok(d.T, int64_t(d.P) * (d.D + 1), kMaxElems) ||
      d.T * d.P > INT32_MAX || d.K > INT32_MAX)
    return FFF_ERROR_INVALID_VALUE;
  *out = d;
  return FFF_SUCCESS;
}

// Deep levels through the token-tile subtree kernel (its records then feed
// the H pass, which needs the whole path: D+1 <= 8).
bool tile_ok(const Dims& s, int k) {
  return k >= 1 && k <= s.D && fff::route_top_supported(s, k) && fff::subtree_supported(s, k) &&
         fff::hbuild_supported(s);
}

// Split levels the prefill algorithm can take for this shape.
bool split_ok(const Dims& s, int k) {
  if (k == s.D + 1) return fff::route_top_supported(s, k);
  return k >= 1 && k <= s.D && fff::route_top_supported(s, k) &&
         (fff::deep_supported(s, k) || tile_ok(s, k));
}

// Up to depth 5 every level is dense: with at most 64 columns per tree the
// dense product beats the token-tile kernel (measured at the GPT-125M shape,
// depth 5: 107 against 72 M tokens/s; OPT-1.3B shape, depth 4: 38 against
// 35 M tokens/s).  At depths 6 and 7 the dense product would evaluate 128 or
// 256 columns per tree for D + 1 nodes on a path; the top D - 3 levels stay
// dense and the last four go through the token-tile kernel (depth 6 at the
// OPT-1.3B shape: 32.6 against 26.7 M tokens/s all dense).  From depth 8 the
// H pass cannot take the whole path's records, and the bucketed kernels take
// the last levels (depth 8 and beyond, measured at T = 16384, d = 2048,
// P = 32, h = 128, ms per forward: D = 8 k = 5 0.75, k = 6 0.79).  A shape a
// kernel does not cover falls back to the next choice.
int default_split(const Dims& s) {
  if (s.D <= 5 && split_ok(s, s.D + 1)) return s.D + 1;
  if (s.D >= 3 && tile_ok(s, s.D - 3)) return s.D - 3;
  if (s.D <= 6 && split_ok(s, s.D + 1)) return s.D + 1;
  const int k = s.D == 7 ? 5 : (s.D - 3 > 1 ? s.D - 3 : 1);
  if (k <= s.D && split_ok(s, k)) return k;
  return split_ok(s, s.D + 1) ? s.D + 1 : -1;
}

bool prefill_fits(const Dims& s) {
  return s.dtype == FFF_DTYPE_BF16 && s.d % 64 == 0 && s.h % 64 == 0 && s.K % 64 == 0 &&
         default_split(s) > 0;
}

// `staged`: the plan is for fff_route, which needs the routing stage on its
// own; AUTO then never picks the fused decode kernel.
fff_status_t resolve_plan(const Dims& s, const fff_plan_t* in, fff_plan_t* out,
                          bool staged = false) {
  fff_plan_t p;
  p.algo = in ? in->algo : FFF_ALGO_AUTO;
  p.split_level = in ? in->split_level : -1;
  p.chunk_tokens = in ? in->chunk_tokens : 0;
  p.flags = in ? in->flags : 0;
  if (p.flags & ~kPlanFlags) return FFF_ERROR_INVALID_VALUE;
  if (p.algo == FFF_ALGO_AUTO) {
    if (!staged && fff::decode_supported(s))
      p.algo = FFF_ALGO_DECODE;
    else
      p.algo = prefill_fits(s) ? FFF_ALGO_PREFILL : FFF_ALGO_GENERIC;
  }
  switch (p.algo) {
    case FFF_ALGO_GENERIC:
      p.split_level = 0;
      p.chunk_tokens = 0;
      break;
    case FFF_ALGO_PREFILL:
      if (!prefill_fits(s)) return FFF_ERROR_NOT_SUPPORTED;
      if (p.split_level < 0) p.split_level = default_split(s);
      if (!split_ok(s, p.split_level)) return FFF_ERROR_NOT_SUPPORTED;
      if (p.chunk_tokens < 0) return FFF_ERROR_INVALID_VALUE;
      if (p.split_level <= s.D) {
        // chunk_tokens 0: the token-tile kernel where it applies (it stays 0
        // in the resolved plan); > 0: bucketing in chunks of that many tokens.
        const bool tile = p.chunk_tokens == 0 && tile_ok(s, p.split_level);
        if (!tile && !fff::deep_supported(s, p.split_level)) return FFF_ERROR_NOT_SUPPORTED;
        if (!tile && p.chunk_tokens == 0)
          p.chunk_tokens = static_cast<int32_t>(fff::deep_chunk(s, p.split_level));
        if (p.chunk_tokens > s.T) p.chunk_tokens = static_cast<int32_t>(s.T > 0 ? s.T : 1);
      } else {
        p.chunk_tokens = 0;
      }
      break;
    case FFF_ALGO_DECODE:
      if (staged || !fff::decode_supported(s)) return FFF_ERROR_NOT_SUPPORTED;
      p.split_level = 0;
      p.chunk_tokens = 0;
      break;
    default:
      return FFF_ERROR_INVALID_VALUE;
  }
  *out = p;
  return FFF_SUCCESS;
}

// Workspace carve-up.  Offsets are multiples of kWsAlign.
//   logits  per (tree, token) fp32 logits of the densely evaluated levels
//           (all D+1 levels on the generic path and the token-tile path)
//   leaf    per (tree, token) int32 node state
//   perm    per (tree, token) int32 token ids grouped by bucket (prefill, k <= D)
//   offs    per (chunk, tree) bucket offsets, 2^k + 1 int32 each
//   cnt     per (chunk, tree, slice) bucket counts, 2^k int32 each
//   H       concatenated tree outputs [T, P*h] in the layer dtype
struct Layout {
  size_t logits = 0, leaf = 0, perm = 0, offs = 0, cnt = 0, H = 0;  // offsets
  bool tile = false;  // deep levels through the token-tile kernel (records of all D+1 levels)
  bool split = false;  // token-tile plan whose dense levels run as two K halves
  size_t part = 0;     // their fp32 logits (split only)
  size_t total = 0;
};

size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

Layout layout_for(const Dims& s, const fff_plan_t& p) {
  if (p.algo == FFF_ALGO_DECODE) {  // the decode kernel carves its own
    Layout L;
    L.total = fff::decode_workspace(s);
    return L;
  }
  const bool prefill = p.algo == FFF_ALGO_PREFILL;
  const bool tile = prefill && p.split_level <= s.D && p.chunk_tokens == 0;
  const int levels = prefill && !tile ? p.split_level : s.D + 1;
  const bool deep = prefill && p.split_level <= s.D && !tile;
  Layout L;
  L.tile = tile;
  size_t off = 0;
  L.logits = off;
  off = align_up(off + size_t(s.T) * s.P * levels * sizeof(float));
  L.leaf = off;
  off = align_up(off + size_t(s.T) * s.P * sizeof(int32_t));
  L.perm = off;
  if (deep) off = align_up(off + size_t(s.T) * s.P * sizeof(int32_t));
  L.offs = off;
  if (deep) {
    const size_t nchunks = (size_t(s.T) + p.chunk_tokens - 1) / p.chunk_tokens;
    off = align_up(off + nchunks * s.P * ((size_t(1) << p.split_level) + 1) * sizeof(int32_t));
  }
  L.cnt = off;
  if (deep) off = align_up(off + fff::bucket_count_bytes(s, p.split_level, p.chunk_tokens));
  L.H = off;
  off = align_up(off + size_t(s.T) * size_t(s.K) * s.esize);
  L.split = tile && fff::route_top_split_wanted(s, p.split_level);
  L.part = off;
  if (L.split) off = align_up(off + fff::route_top_split_bytes(s, p.split_level));
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Pruning table carve-up (offsets are multiples of kWsAlign), for L packed
// dense levels (0: alive flags only).  At most P tiles: a tree has fewer
// than 256 columns of levels < L <= 8.
//   alive       [P][N] uint8
//   tree_base   [P] int32            first column of tree p within its tile
//   tile_first  [P] int32, tile_count [P] int32
//   colmap      [P * 256] int32      source row p*N + n of each packed column, -1 = zero row
//   colinfo     [P * 256] uint32     children of each packed column (tile columns, alive bits)
//   packed      [P * 256][d] bf16
struct PruneLayout {
  size_t alive = 0, tree_base = 0, tile_first = 0, tile_count = 0, colmap = 0,
         colinfo = 0, packed = 0, total = 0;
};

PruneLayout prune_layout(const Dims& s, int L) {
  PruneLayout PL;
  size_t off = 0;
  PL.alive = off;
  off = align_up(off + size_t(s.P) * size_t(s.N));
  if (L > 0) {
    PL.tree_base = off;
    off = align_up(off + size_t(s.P) * sizeof(int32_t));
    PL.tile_first = off;
    off = align_up(off + size_t(s.P) * sizeof(int32_t));
    PL.tile_count = off;
    off = align_up(off + size_t(s.P) * sizeof(int32_t));
    PL.colmap = off;
    off = align_up(off + size_t(s.P) * 256 * sizeof(int32_t));
    PL.colinfo = off;
    off = align_up(off + size_t(s.P) * 256 * sizeof(uint32_t));
    PL.packed = off;
    off = align_up(off + size_t(s.P) * 256 * size_t(s.d) * 2);
  }
  PL.total = off;
  return PL;
}

int packed_levels(const fff_plan_t& p) { return p.algo == FFF_ALGO_PREFILL ? p.split_level : 0; }

fff_status_t hip_status(hipError_t e) { return e == hipSuccess ? FFF_SUCCESS : FFF_ERROR_HIP; }

fff_status_t record(hipEvent_t ev, hipStream_t st) {
  if (!ev) return FFF_SUCCESS;
  return hip_status(hipEventRecord(ev, st));
}

// Whether the routing stage of a plan writes H through hbuild_kernel (the
// dense and token-tile prefill plans) and the direct-to-LDS projection takes
// it: then fff_forward keeps H K-blocked, so that each projection stage
// reads whole 128-byte lines.
bool h_blocked(const Dims& s, const fff_plan_t& p, const Layout& L) {
  return p.algo == FFF_ALGO_PREFILL && (L.tile || p.split_level == s.D + 1) &&
         fff::project_direct_supported(s);
}

// Routing stage into H (caller or workspace buffer; K-blocked with
// `blocked`, which needs a plan for which h_blocked() holds); records the
// `top` and `deep` events (NULL events: none).
fff_status_t run_route(const Dims& s, const fff_plan_t& p, const Layout& L, const void* x,
                       const void* W, const void* b, const void* V, void* H, int32_t* path_out,
                       char* ws, bool blocked, hipStream_t st, const fff_stage_events_t* ev) {
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* leaf = reinterpret_cast<int32_t*>(ws + L.leaf);
  const fff_stage_events_t none{};
  const fff_stage_events_t& E = ev ? *ev : none;
  hipError_t e;
  fff_status_t r;
  if (p.algo == FFF_ALGO_PREFILL) {
    const int k = p.split_level;
    if (L.split) {
      // Dense levels as two K halves; the token-tile kernel walks them.
      float* part = reinterpret_cast<float*>(ws + L.part);
      e = fff::launch_route_top_split(s, k, x, W, part, st);
      if (e != hipSuccess) return FFF_ERROR_HIP;
      if ((r = record(E.top, st)) != FFF_SUCCESS) return r;
      e = fff::launch_subtree(s, k, x, W, b, logits, leaf, part,
                              fff::route_top_split_cols(s, k), st);
      if (e != hipSuccess) return FFF_ERROR_HIP;
      if ((r = record(E.deep, st)) != FFF_SUCCESS) return r;
      return hip_status(fff::launch_hbuild(s, logits, leaf, V, H, path_out, blocked, st));
    }
    e = fff::launch_route_top(s, k, L.tile ? s.D + 1 : k, x, W, b, logits, leaf, st);
    if (e != hipSuccess) return FFF_ERROR_HIP;
    if ((r = record(E.top, st)) != FFF_SUCCESS) return r;
    if (k == s.D + 1) {
      if ((r = record(E.deep, st)) != FFF_SUCCESS) return r;
      return hip_status(fff::launch_hbuild(s, logits, leaf, V, H, path_out, blocked, st));
    }
    if (L.tile) {
      e = fff::launch_subtree(s, k, x, W, b, logits, leaf, nullptr, 0, st);
      if (e != hipSuccess) return FFF_ERROR_HIP;
      if ((r = record(E.deep, st)) != FFF_SUCCESS) return r;
      return hip_status(fff::launch_hbuild(s, logits, leaf, V, H, path_out, blocked, st));
    }
    int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
    int32_t* offs = reinterpret_cast<int32_t*>(ws + L.offs);
    int32_t* cnt = reinterpret_cast<int32_t*>(ws + L.cnt);
    e = fff::launch_bucket(s, k, leaf, perm, offs, cnt, p.chunk_tokens, st);
    if (e != hipSuccess) return FFF_ERROR_HIP;
    e = fff::launch_deep(s, k, x, W, b, V, logits, perm, offs, H, path_out, p.chunk_tokens, st);
    if (e != hipSuccess) return FFF_ERROR_HIP;
    return record(E.deep, st);  // the deep kernel writes H itself
  }
  e = fff::launch_route_generic(s, x, W, b, logits, path_out, leaf, st);
  if (e != hipSuccess) return FFF_ERROR_HIP;
  if ((r = record(E.top, st)) != FFF_SUCCESS) return r;
  if ((r = record(E.deep, st)) != FFF_SUCCESS) return r;
  e = fff::launch_hbuild_generic(s, logits, leaf, V, H, st);
  return hip_status(e);
}

fff_status_t run_project(const Dims& s, int32_t algo, const void* H, const void* Wout, void* y,
                         hipStream_t st) {
  hipError_t e;
  if (algo != FFF_ALGO_GENERIC && fff::project_direct_supported(s))
    e = fff::launch_project_direct(s, H, Wout, y, false, st);
  else if (algo != FFF_ALGO_GENERIC && fff::project_mfma_supported(s))
    e = fff::launch_project_mfma(s, H, Wout, y, st);
  else
    e = fff::launch_project_generic(s, H, Wout, y, st);
  return hip_status(e);
}

// fff_project_ws: every projection kernel reads W_out in its own layout, so
// none needs workspace.
size_t project_ws_bytes(const Dims&, int32_t) { return 0; }

fff_status_t check_inputs(const Dims& s, const void* x, const void* W, const void* b,
                          const void* V) {
  if (!x || !W || !b || !V) return FFF_ERROR_INVALID_VALUE;
  if (!aligned(x, 16) || !aligned(W, 16) || !aligned(V, 16) || !aligned(b, s.esize))
    return FFF_ERROR_INVALID_VALUE;
  return FFF_SUCCESS;
}

// The whole layer for a validated shape and resolved plan (s.prune set for
// pruned trees).
fff_status_t forward_impl(const Dims& s, const fff_plan_t& p, const void* x, const void* W_node,
                          const void* b_node, const void* V_node, const void* W_out, void* y,
                          int32_t* path_out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream, const fff_stage_events_t* events) {
  fff_status_t st;
  if (s.T == 0) return FFF_SUCCESS;
  st = check_inputs(s, x, W_node, b_node, V_node);
  if (st != FFF_SUCCESS) return st;
  if (!W_out || !y || !aligned(W_out, 16) || !aligned(y, 16) ||
      (path_out && !aligned(path_out, 4)))
    return FFF_ERROR_INVALID_VALUE;
  const Layout L = layout_for(s, p);
  if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return FFF_ERROR_WORKSPACE;
  if (workspace && !aligned(workspace, kWsAlign)) return FFF_ERROR_INVALID_VALUE;

  char* ws = static_cast<char*>(workspace);
  void* H = ws + L.H;
  const fff_stage_events_t none{};
  const fff_stage_events_t& E = events ? *events : none;
  if ((st = record(E.start, stream)) != FFF_SUCCESS) return st;
  if (p.algo == FFF_ALGO_DECODE) {
    st = hip_status(fff::launch_decode(s, x, W_node, b_node, V_node, W_out, y, path_out, ws,
                                       p.flags, stream));
    if (st != FFF_SUCCESS) return st;
    for (hipEvent_t ev : {E.prepared, E.top, E.deep, E.routed, E.done})
      if ((st = record(ev, stream)) != FFF_SUCCESS) return st;
    return FFF_SUCCESS;
  }
  // Nothing is prepared before routing (W_out is used in its own layout):
  // `prepared` follows `start` directly.
  if ((st = record(E.prepared, stream)) != FFF_SUCCESS) return st;
  const bool blk = h_blocked(s, p, L);
  st = run_route(s, p, L, x, W_node, b_node, V_node, H, path_out, ws, blk, stream, &E);
  if (st != FFF_SUCCESS) return st;
  if ((st = record(E.routed, stream)) != FFF_SUCCESS) return st;
  if (blk)
    st = hip_status(fff::launch_project_direct(s, H, W_out, y, true, stream));
  else
    st = run_project(s, p.algo, H, W_out, y, stream);
  if (st != FFF_SUCCESS) return st;
  if ((st = record(E.done, stream)) != FFF_SUCCESS) return st;
  return FFF_SUCCESS;
}

// ---- backward ----

bool bwd_mfma_fits(const Dims& s) { return fff::backward_mfma_supported(s); }

// A pruned backward (pruning non-null) runs on the matrix cores only with a
// table whose dense levels are all D + 1 levels: its routing is the dense
// product over the packed alive rows.
fff_status_t resolve_bwd_plan(const Dims& s, const fff_plan_t* in, fff_plan_t* out,
                              const fff_pruning_t* pruning = nullptr) {
  fff_plan_t p;
  p.algo = in ? in->algo : FFF_ALGO_AUTO;
  p.split_level = in ? in->split_level : -1;
  p.chunk_tokens = 0;
  p.flags = in ? in->flags : 0;
  if (p.flags & ~kPlanFlags) return FFF_ERROR_INVALID_VALUE;
  const bool table_ok = !pruning || pruning->split_level == s.D + 1;
  if (p.algo == FFF_ALGO_AUTO)
    p.algo = bwd_mfma_fits(s) && table_ok ? FFF_ALGO_PREFILL : FFF_ALGO_GENERIC;
  switch (p.algo) {
    case FFF_ALGO_GENERIC:
      p.split_level = 0;
      break;
    case FFF_ALGO_PREFILL:
      if (!bwd_mfma_fits(s) || !table_ok || (p.split_level >= 0 && p.split_level != s.D + 1))
        return FFF_ERROR_NOT_SUPPORTED;
      p.split_level = s.D + 1;
      break;
    case FFF_ALGO_DECODE:
      return FFF_ERROR_NOT_SUPPORTED;
    default:
      return FFF_ERROR_INVALID_VALUE;
  }
  *out = p;
  return FFF_SUCCESS;
}

// Backward workspace (generic plan):
//   logits [T][P][D+1] f32, leaf [T][P] i32, dH [T][K] f32, H [T][K] f32,
//   dx accumulator [T][d] f32.
struct BwdLayout {
  size_t logits = 0, leaf = 0, dH = 0, H = 0, dxacc = 0, total = 0;
};

BwdLayout bwd_layout(const Dims& s, const fff_plan_t& p) {
  BwdLayout B;
  if (p.algo == FFF_ALGO_PREFILL) {
    B.total = s.T == 0 ? 0 : fff::backward_mfma_layout(s).total;
    return B;
  }
  size_t off = 0;
  B.logits = off;
  off = align_up(off + size_t(s.T) * s.P * (s.D + 1) * 4);
  B.leaf = off;
  off = align_up(off + size_t(s.T) * s.P * 4);
  B.dH = off;
  off = align_up(off + size_t(s.T) * size_t(s.K) * 4);
  B.H = off;
  off = align_up(off + size_t(s.T) * size_t(s.K) * 4);
  B.dxacc = off;
  off = align_up(off + size_t(s.T) * s.d * 4);
  B.total = s.T == 0 ? 0 : off;
  return B;
}

// The device views of a prepared pruning table, after checking that it was
// prepared for this shape's trees.
fff_status_t prune_view(const Dims& s, const fff_pruning_t* pruning, fff::PruneView* pv) {
  if (!pruning || !pruning->table || !aligned(pruning->table, kWsAlign) || pruning->P != s.P ||
      pruning->D != s.D || pruning->d != s.d || pruning->split_level < 0 ||
      pruning->split_level > 8 || pruning->col_tiles < 0 || pruning->col_tiles > s.P ||
      (pruning->split_level > 0 && pruning->col_tiles < 1))  // packed levels need a tile
    return FFF_ERROR_INVALID_VALUE;
  const PruneLayout PL = prune_layout(s, pruning->split_level);
  const char* tb = static_cast<const char*>(pruning->table);
  *pv = fff::PruneView{};
  pv->alive = reinterpret_cast<const uint8_t*>(tb + PL.alive);
  if (pruning->split_level > 0) {
    pv->tree_base = reinterpret_cast<const int32_t*>(tb + PL.tree_base);
    pv->tile_first = reinterpret_cast<const int32_t*>(tb + PL.tile_first);
    pv->tile_count = reinterpret_cast<const int32_t*>(tb + PL.tile_count);
    pv->colmap = reinterpret_cast<const int32_t*>(tb + PL.colmap);
    pv->colinfo = reinterpret_cast<const uint32_t*>(tb + PL.colinfo);
    pv->W_packed = reinterpret_cast<const uint16_t*>(tb + PL.packed);
  }
  pv->L = pruning->split_level;
  pv->col_tiles = pruning->col_tiles;
  return FFF_SUCCESS;
}

// The backward pass for a validated shape (s.prune set for pruned trees)
// and resolved plan.
fff_status_t backward_impl(const Dims& s, const fff_plan_t& p, const void* x, const void* W_node,
                           const void* b_node, const void* V_node, const void* W_out,
                           const void* dy, void* dx, float* dW_node, float* db_node,
                           float* dV_node, float* dW_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!dW_node || !db_node || !dV_node || !dW_out || !aligned(dW_node, 16) ||
      !aligned(db_node, 4) || !aligned(dV_node, 16) || !aligned(dW_out, 16))
    return FFF_ERROR_INVALID_VALUE;
  const int64_t nW = int64_t(s.P) * s.N * s.d, nb = int64_t(s.P) * s.N;
  const int64_t nV = int64_t(s.P) * s.N * s.h, nO = s.K * s.d;
  if (s.T == 0) {  // no token: every gradient is zero
    if (fff::launch_fill_f32(dW_node, nW, stream) != hipSuccess ||
        fff::launch_fill_f32(db_node, nb, stream) != hipSuccess ||
        fff::launch_fill_f32(dV_node, nV, stream) != hipSuccess ||
        fff::launch_fill_f32(dW_out, nO, stream) != hipSuccess)
      return FFF_ERROR_HIP;
    return FFF_SUCCESS;
  }
  fff_status_t st = check_inputs(s, x, W_node, b_node, V_node);
  if (st != FFF_SUCCESS) return st;
  if (!W_out || !dy || !dx || !aligned(W_out, 16) || !aligned(dy, 16) || !aligned(dx, 16))
    return FFF_ERROR_INVALID_VALUE;
  const BwdLayout B = bwd_layout(s, p);
  if (!workspace || workspace_bytes < B.total) return FFF_ERROR_WORKSPACE;
  if (!aligned(workspace, kWsAlign)) return FFF_ERROR_INVALID_VALUE;
  if (p.algo == FFF_ALGO_PREFILL)
    return hip_status(fff::launch_backward_mfma(s, x, W_node, b_node, V_node, W_out, dy, dx,
                                                dW_node, db_node, dV_node, dW_out, workspace,
                                                stream));
  char* ws = static_cast<char*>(workspace);
  float* logits = reinterpret_cast<float*>(ws + B.logits);
  int32_t* leaf = reinterpret_cast<int32_t*>(ws + B.leaf);
  if (fff::launch_route_generic(s, x, W_node, b_node, logits, nullptr, leaf, stream) != hipSuccess)
    return FFF_ERROR_HIP;
  return hip_status(fff::launch_backward_generic(
      s, x, W_node, V_node, W_out, dy, dx, dW_node, db_node, dV_node, dW_out, logits, leaf,
      reinterpret_cast<float*>(ws + B.dH), reinterpret_cast<float*>(ws + B.H),
      reinterpret_cast<float*>(ws + B.dxacc), stream));
}

}  // namespace

extern "C" {

fff_status_t fff_backward_workspace_size(const fff_shape_t* shape, const fff_plan_t* plan,
                                         size_t* bytes) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  if (!bytes) return FFF_ERROR_INVALID_VALUE;
  fff_plan_t p;
  st = resolve_bwd_plan(s, plan, &p);
  if (st != FFF_SUCCESS) return st;
  *bytes = bwd_layout(s, p).total;
  return FFF_SUCCESS;
}

fff_status_t fff_backward(const fff_shape_t* shape, const fff_plan_t* plan, const void* x,
                          const void* W_node, const void* b_node, const void* V_node,
                          const void* W_out, const void* dy, void* dx, float* dW_node,
                          float* db_node, float* dV_node, float* dW_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  fff_plan_t p;
  st = resolve_bwd_plan(s, plan, &p);
  if (st != FFF_SUCCESS) return st;
  return backward_impl(s, p, x, W_node, b_node, V_node, W_out, dy, dx, dW_node, db_node, dV_node,
                       dW_out, workspace, workspace_bytes, stream);
}

fff_status_t fff_backward_pruned_workspace_size(const fff_shape_t* shape, const fff_plan_t* plan,
                                                const fff_pruning_t* pruning, size_t* bytes) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  if (!bytes) return FFF_ERROR_INVALID_VALUE;
  fff::PruneView pv;
  st = prune_view(s, pruning, &pv);
  if (st != FFF_SUCCESS) return st;
  fff_plan_t p;
  st = resolve_bwd_plan(s, plan, &p, pruning);
  if (st != FFF_SUCCESS) return st;
  *bytes = bwd_layout(s, p).total;
  return FFF_SUCCESS;
}

fff_status_t fff_backward_pruned(const fff_shape_t* shape, const fff_plan_t* plan,
                                 const fff_pruning_t* pruning, const void* x, const void* W_node,
                                 const void* b_node, const void* V_node, const void* W_out,
                                 const void* dy, void* dx, float* dW_node, float* db_node,
                                 float* dV_node, float* dW_out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  fff::PruneView pv;
  st = prune_view(s, pruning, &pv);
  if (st != FFF_SUCCESS) return st;
  fff_plan_t p;
  st = resolve_bwd_plan(s, plan, &p, pruning);
  if (st != FFF_SUCCESS) return st;
  s.prune = &pv;
  return backward_impl(s, p, x, W_node, b_node, V_node, W_out, dy, dx, dW_node, db_node, dV_node,
                       dW_out, workspace, workspace_bytes, stream);
}

}  // extern "C"

extern "C" {

fff_status_t fff_plan_default(const fff_shape_t* shape, fff_plan_t* plan) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  if (!plan) return FFF_ERROR_INVALID_VALUE;
  return resolve_plan(s, nullptr, plan);
}

fff_status_t fff_plan_resolve(const fff_shape_t* shape, const fff_plan_t* in, fff_plan_t* out) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  if (!in || !out) return FFF_ERROR_INVALID_VALUE;
  return resolve_plan(s, in, out);
}

fff_status_t fff_workspace_size(const fff_shape_t* shape, const fff_plan_t* plan, size_t* bytes) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  if (!bytes) return FFF_ERROR_INVALID_VALUE;
  fff_plan_t p;
  st = resolve_plan(s, plan, &p);
  if (st != FFF_SUCCESS) return st;
  size_t n = layout_for(s, p).total;
  // The same plan given to fff_route may resolve to a staged algorithm.
  fff_plan_t pr;
  if (resolve_plan(s, plan, &pr, true) == FFF_SUCCESS) {
    const size_t nr = layout_for(s, pr).total;
    if (nr > n) n = nr;
  }
  *bytes = s.T == 0 ? 0 : n;
  return FFF_SUCCESS;
}

fff_status_t fff_forward(const fff_shape_t* shape, const fff_plan_t* plan, const void* x,
                         const void* W_node, const void* b_node, const void* V_node,
                         const void* W_out, void* y, int32_t* path_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream,
                         const fff_stage_events_t* events) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  fff_plan_t p;
  st = resolve_plan(s, plan, &p);
  if (st != FFF_SUCCESS) return st;
  return forward_impl(s, p, x, W_node, b_node, V_node, W_out, y, path_out, workspace,
                      workspace_bytes, stream, events);
}

fff_status_t fff_prune_table_size(const fff_shape_t* shape, const fff_plan_t* plan,
                                  size_t* bytes) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  if (!bytes) return FFF_ERROR_INVALID_VALUE;
  fff_plan_t p;
  st = resolve_plan(s, plan, &p);
  if (st != FFF_SUCCESS) return st;
  *bytes = prune_layout(s, packed_levels(p)).total;
  return FFF_SUCCESS;
}

fff_status_t fff_prune_prepare(const fff_shape_t* shape, const fff_plan_t* plan,
                               const uint8_t* leaf_alive, const void* W_node, void* table,
                               size_t table_bytes, hipStream_t stream, fff_pruning_t* out) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  fff_plan_t p;
  st = resolve_plan(s, plan, &p);
  if (st != FFF_SUCCESS) return st;
  if (!leaf_alive || !W_node || !table || !out || !aligned(table, kWsAlign) ||
      !aligned(W_node, 16))
    return FFF_ERROR_INVALID_VALUE;
  if (int64_t(s.P) * s.N > INT32_MAX) return FFF_ERROR_NOT_SUPPORTED;
  const int L = packed_levels(p);
  const PruneLayout PL = prune_layout(s, L);
  if (table_bytes < PL.total) return FFF_ERROR_WORKSPACE;

  // Node flags: leaves as given, internal nodes alive iff a child is.
  const int64_t N = s.N;
  const int64_t first_leaf = (int64_t(1) << s.D) - 1;
  std::vector<uint8_t> alive(size_t(s.P) * N);
  for (int64_t t = 0; t < s.P; ++t) {
    uint8_t* a = alive.data() + t * N;
    for (int64_t i = 0; i <= first_leaf; ++i) a[first_leaf + i] = leaf_alive[t * (first_leaf + 1) + i] != 0;
    for (int64_t n = first_leaf - 1; n >= 0; --n) a[n] = a[2 * n + 1] | a[2 * n + 2];
    if (!a[0]) return FFF_ERROR_INVALID_VALUE;
  }
  // Packed columns of the dense levels: trees in order, a new tile when the
  // next tree does not fit; within a tree, alive nodes in heap order.
  const int64_t cols = L > 0 ? (int64_t(1) << L) - 1 : 0;
  std::vector<int16_t> colidx(size_t(s.P) * cols, -1);
  std::vector<int32_t> tree_base(s.P, 0), tile_first(s.P, 0), tile_count(s.P, 0);
  std::vector<int32_t> colmap(size_t(s.P) * 256, -1);
  int tiles = 0;
  if (L > 0) {
    int used = 256;
    for (int t = 0; t < s.P; ++t) {
      int cnt = 0;
      for (int64_t n = 0; n < cols; ++n) cnt += alive[t * N + n];
      if (used + cnt > 256) {
        tile_first[tiles] = t;
        ++tiles;
        used = 0;
      }
      tree_base[t] = used;
      ++tile_count[tiles - 1];
      int i = 0;
      for (int64_t n = 0; n < cols; ++n) {
        if (!alive[t * N + n]) continue;
        colidx[t * cols + n] = static_cast<int16_t>(i);
        colmap[size_t(tiles - 1) * 256 + used + i] = static_cast<int32_t>(t * N + n);
        ++i;
      }
      used += cnt;
    }
  }
  // Children of every packed column: their columns in the tile (when they
  // are dense too) and whether they are alive.
  std::vector<uint32_t> colinfo(size_t(s.P) * 256, 0);
  for (size_t c = 0; c < colmap.size(); ++c) {
    if (colmap[c] < 0) continue;
    const int64_t t = colmap[c] / N;
    const int64_t n = colmap[c] - t * N;
    if (n >= first_leaf) continue;  // a leaf: no children
    uint32_t info = 0;
    for (int r = 0; r < 2; ++r) {
      const int64_t ch = 2 * n + 1 + r;
      if (!alive[t * N + ch]) continue;
      info |= 1u << (18 + r);
      if (ch < cols) info |= uint32_t(tree_base[t] + colidx[t * cols + ch]) << (9 * r);
    }
    colinfo[c] = info;
  }
  char* tb = static_cast<char*>(table);
  auto put = [&](size_t off, const void* src, size_t n) {
    return n == 0 || hipMemcpyAsync(tb + off, src, n, hipMemcpyHostToDevice, stream) == hipSuccess;
  };
  bool ok = put(PL.alive, alive.data(), alive.size());
  if (L > 0) {
    ok = ok && put(PL.tree_base, tree_base.data(), tree_base.size() * sizeof(int32_t)) &&
         put(PL.tile_first, tile_first.data(), tile_first.size() * sizeof(int32_t)) &&
         put(PL.tile_count, tile_count.data(), tile_count.size() * sizeof(int32_t)) &&
         put(PL.colmap, colmap.data(), colmap.size() * sizeof(int32_t)) &&
         put(PL.colinfo, colinfo.data(), colinfo.size() * sizeof(uint32_t)) &&
         fff::launch_prune_pack(W_node, reinterpret_cast<const int32_t*>(tb + PL.colmap),
                                tb + PL.packed, tiles * 256, s.d, stream) == hipSuccess;
  }
  // The host vectors above are the copies' sources: wait before they go.
  if (hipStreamSynchronize(stream) != hipSuccess || !ok) return FFF_ERROR_HIP;
  out->table = table;
  out->P = s.P;
  out->D = s.D;
  out->d = s.d;
  out->split_level = L;
  out->col_tiles = tiles;
  return FFF_SUCCESS;
}

fff_status_t fff_forward_pruned(const fff_shape_t* shape, const fff_plan_t* plan,
                                const fff_pruning_t* pruning, const void* x, const void* W_node,
                                const void* b_node, const void* V_node, const void* W_out,
                                void* y, int32_t* path_out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream,
                                const fff_stage_events_t* events) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  fff::PruneView pv;
  st = prune_view(s, pruning, &pv);
  if (st != FFF_SUCCESS) return st;
  fff_plan_t p;
  st = resolve_plan(s, plan, &p);
  if (st != FFF_SUCCESS) return st;
  if (p.algo == FFF_ALGO_PREFILL && p.split_level != pruning->split_level)
    return FFF_ERROR_NOT_SUPPORTED;
  s.prune = &pv;
  return forward_impl(s, p, x, W_node, b_node, V_node, W_out, y, path_out, workspace,
                      workspace_bytes, stream, events);
}

fff_status_t fff_route(const fff_shape_t* shape, const fff_plan_t* plan, const void* x,
                       const void* W_node, const void* b_node, const void* V_node, void* H,
                       int32_t* path_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  fff_plan_t p;
  st = resolve_plan(s, plan, &p, true);
  if (st != FFF_SUCCESS) return st;
  if (s.T == 0) return FFF_SUCCESS;
  st = check_inputs(s, x, W_node, b_node, V_node);
  if (st != FFF_SUCCESS) return st;
  if (!H || !aligned(H, 16) || (path_out && !aligned(path_out, 4))) return FFF_ERROR_INVALID_VALUE;
  const Layout L = layout_for(s, p);
  if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return FFF_ERROR_WORKSPACE;
  if (workspace && !aligned(workspace, kWsAlign)) return FFF_ERROR_INVALID_VALUE;
  // fff_route hands H to the caller: row-major, as fff.h documents it.
  return run_route(s, p, L, x, W_node, b_node, V_node, H, path_out, static_cast<char*>(workspace),
                   false, stream, nullptr);
}

fff_status_t fff_project(const fff_shape_t* shape, int32_t algo, const void* H, const void* W_out,
                         void* y, hipStream_t stream) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  if (algo != FFF_ALGO_AUTO && algo != FFF_ALGO_GENERIC && algo != FFF_ALGO_PREFILL)
    return FFF_ERROR_INVALID_VALUE;
  if (algo == FFF_ALGO_PREFILL && !fff::project_mfma_supported(s)) return FFF_ERROR_NOT_SUPPORTED;
  if (s.T == 0) return FFF_SUCCESS;
  if (!H || !W_out || !y || !aligned(H, 16) || !aligned(W_out, 16) || !aligned(y, 16))
    return FFF_ERROR_INVALID_VALUE;
  return run_project(s, algo, H, W_out, y, stream);
}

fff_status_t fff_project_workspace_size(const fff_shape_t* shape, int32_t algo, size_t* bytes) {
  if (!bytes) return FFF_ERROR_INVALID_VALUE;
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  if (algo != FFF_ALGO_AUTO && algo != FFF_ALGO_GENERIC && algo != FFF_ALGO_PREFILL)
    return FFF_ERROR_INVALID_VALUE;
  *bytes = project_ws_bytes(s, algo);
  return FFF_SUCCESS;
}

fff_status_t fff_project_ws(const fff_shape_t* shape, int32_t algo, const void* H,
                            const void* W_out, void* y, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  Dims s;
  fff_status_t st = check_shape(shape, &s);
  if (st != FFF_SUCCESS) return st;
  if (algo != FFF_ALGO_AUTO && algo != FFF_ALGO_GENERIC && algo != FFF_ALGO_PREFILL)
    return FFF_ERROR_INVALID_VALUE;
  if (algo == FFF_ALGO_PREFILL && !fff::project_mfma_supported(s)) return FFF_ERROR_NOT_SUPPORTED;
  if (s.T == 0) return FFF_SUCCESS;
  if (!H || !W_out || !y || !aligned(H, 16) || !aligned(W_out, 16) || !aligned(y, 16))
    return FFF_ERROR_INVALID_VALUE;
  (void)workspace;  // no projection kernel needs one (project_ws_bytes is 0)
  (void)workspace_bytes;
  return run_project(s, algo, H, W_out, y, stream);
}

const char* fff_status_string(fff_status_t status) {
  switch (status) {
    case FFF_SUCCESS:
      return "success";
    case FFF_ERROR_INVALID_VALUE:
      return "invalid value (shape, null or misaligned pointer)";
    case FFF_ERROR_NOT_SUPPORTED:
      return "not supported (dtype or plan)";
    case FFF_ERROR_WORKSPACE:
      return "workspace missing or too small";
    case FFF_ERROR_HIP:
      return "HIP runtime or launch error";
  }
  return "unknown status";
}

const char* fff_algo_name(int32_t algo) {
  switch (algo) {
    case FFF_ALGO_AUTO:
      return "auto";
    case FFF_ALGO_GENERIC:
      return "generic";
    case FFF_ALGO_PREFILL:
      return "prefill";
    case FFF_ALGO_DECODE:
      return "decode";
  }
  return "unknown";
}

}  // extern "C"
