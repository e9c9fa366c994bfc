// Routing of the FFF layer on gfx950: the top tree levels as one dense
// matrix-core product, the walk over them, and the GELU * v accumulation.
//
// The FFF explainer page (gist.science, section 2, Implementation) describes
// a "masked" evaluation: all node logits computed in parallel, then a binary
// tree search picks the path.  route_top_kernel does exactly that for the
// first L levels of every tree: with cpt = 2^L columns per tree (nodes
// 0 .. 2^L - 2 in heap order plus one unused column) it computes
//     A[t, (p, n)] = x[t, :] . W_node[p, n, :]          (bf16 MFMA, fp32 acc)
// for a 256-token x 256-column tile, stages the fp32 tile in LDS, and walks
// each (token, tree) over those L levels: a = A + b_node, left iff a < 0.
// It records the L logits and the node reached, per tree and token:
//     rec_logit[p][t][l]   (fp32, l < L)
//     rec_next[p][t]       (heap id at level L, or the leaf if L = D+1)
//
// With static path pruning (a leaf mask per tree, paper page Figure 4) the
// B operand is the table's packed alive rows instead: whole trees per
// 256-column tile, a per-tree column map, and a step into a pruned child
// goes to its sibling.
//
// When L = D+1 the whole path is known and hbuild_kernel forms
//     H[t, p*h + j] = sum over l of GELU(a_l) * V_node[p, n_l, j]
// (GELU before the sum: explainer section 3.C) and path_out; otherwise the
// deep levels continue per token bucket in k_deep.hip.
#include "common.hpp"
#include "launch.hpp"
#include "mfma_tile.hpp"

namespace fff {
namespace {

using TopTile = TileCfg<256, 256, 64, 128, 128>;

// A operand: rows of x, clamped to T-1.
template <class C>
struct XLoader {
  RowLoader<C::BM, C::BK, C::kThreads> rl;
  const uint16_t* x;
  int d, T, m0, tid;
  __device__ __forceinline__ void load(int k0) {
    rl.load([&](int i) {
      const int r = m0 + i < T ? m0 + i : T - 1;
      return x + static_cast<size_t>(r) * d;
    }, k0, tid);
  }
  __device__ __forceinline__ void store(uint16_t* lds, int ld) const { rl.store(lds, ld, tid); }
};

// B operand: one W_node row per column (p, n).  Unused columns (the spare
// column of each tree, trees past P) read row (0, 0); their results are
// never used.
template <class C>
struct NodeRowLoader {
  RowLoader<C::BN, C::BK, C::kThreads> rl;
  const uint16_t* W;
  const uint16_t* packed;  // pruned: the table's packed rows, else null
  int d, P, L, n0, tid;
  int64_t N;
  __device__ __forceinline__ void load(int k0) {
    rl.load([&](int i) {
      if (packed) return packed + static_cast<int64_t>(n0 + i) * d;
      const int gc = n0 + i;
      const int p = gc >> L;
      const int n = gc & ((1 << L) - 1);
      const bool used = p < P && n < (1 << L) - 1;
      return W + (used ? (static_cast<int64_t>(p) * N + n) * d : 0);
    }, k0, tid);
  }
  __device__ __forceinline__ void store(uint16_t* lds, int ld) const { rl.store(lds, ld, tid); }
};

// Walk epilogue shared by the top-level kernels.  acc holds the tile's
// logits without bias (transposed-block layout of mfma_tile.hpp); `lg` is
// LDS of at least WM * (BN + 4) + 2 * BN floats, free for reuse.
// Per tile column: the node's bias and, pruned, its children's columns and
// alive flags.  Thread c < BN loads column c before the main loop so that
// the loads are long done when the epilogue stages them.
struct ColMeta {
  float bias;
  uint32_t info;
};
template <class C>
__device__ __forceinline__ ColMeta load_col_meta(const uint16_t* __restrict__ b, int P, int L,
                                                 int64_t N, int n0, const PruneView& pv) {
  static_assert(C::kThreads >= C::BN, "one thread per tile column");
  ColMeta cm{0.0f, 0u};
  const int c = threadIdx.x;
  if (c < C::BN) {
    int64_t g = -1;  // heap row p*N + n of column c
    if (pv.alive) {
      g = pv.colmap[n0 + c];
      cm.info = pv.colinfo[n0 + c];
    } else {
      const int cpt = 1 << L;
      const int p = (n0 + c) >> L;
      const int n = (n0 + c) & (cpt - 1);
      if (p < P && n < cpt - 1) g = static_cast<int64_t>(p) * N + n;
    }
    cm.bias = g >= 0 ? bf16_to_f32(b[g]) : 0.0f;
  }
  return cm;
}

template <class C>
__device__ __forceinline__ void top_walk_epilogue(const f32x16_t (&acc)[C::kTm][C::kTn], float* lg,
                                                  const ColMeta& cm,
                                                  float* __restrict__ rec_logit,
                                                  int32_t* __restrict__ rec_next, int T, int P,
                                                  int D, int L, int stride, int64_t N, int m0,
                                                  int n0, const PruneView& pv) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / C::kWavesN;
  const int wn = wave % C::kWavesN;
  // Two passes of WM token rows each (the fp32 tile of one pass, WM x BN,
  // fits in the LDS freed by the main loop).
  constexpr int kRows = C::WM;
  constexpr int kPitch = C::BN + 4;
  const int cpt = 1 << L;
  // Trees of this column tile (consecutive ids).  Unpruned: BN >> L trees of
  // cpt columns each; pruned: as the table packed them.
  const int tn = n0 / C::BN;
  const int tpt = pv.alive ? pv.tile_count[tn] : C::BN >> L;
  const int p_base = pv.alive ? pv.tile_first[tn] : n0 >> L;
  // Per column of the tile: its node's bias and, pruned, its children's
  // columns and alive flags; staged once so that the walks below read no
  // global memory per level (visible after the first pass's barrier).
  float* bias_s = lg + kRows * kPitch;
  uint32_t* info_s = reinterpret_cast<uint32_t*>(bias_s + C::BN);
  if (tid < C::BN) {
    bias_s[tid] = cm.bias;
    info_s[tid] = cm.info;
  }
#pragma unroll 1
  for (int half = 0; half < C::kWavesM; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < C::kTm; ++i)
#pragma unroll
        for (int j = 0; j < C::kTn; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int row = i * 32 + (lane & 31);
            const int col = wn * C::WN + j * 32 + g * 8 + (lane >> 5) * 4;
            *reinterpret_cast<float4*>(lg + row * kPitch + col) =
                make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                            acc[i][j][4 * g + 3]);
          }
    }
    __syncthreads();
    for (int q = tid; q < kRows * tpt; q += C::kThreads) {
      const int tr = q % kRows;
      const int tp = q / kRows;
      const int t = m0 + half * kRows + tr;
      const int p = p_base + tp;
      if (t >= T || p >= P) continue;
      float* out = rec_logit + (static_cast<int64_t>(p) * T + t) * stride;
      const float* row = lg + tr * kPitch;
      int n = 0;
      if (!pv.alive) {
        const int c0 = tp * cpt;  // node n at column c0 + n
        for (int level = 0; level < L; ++level) {
          const float a = row[c0 + n] + bias_s[c0 + n];
          out[level] = a;
          if (level < D) n = 2 * n + 1 + go_right(a);
        }
      } else {
        // Packed columns: the root at the tree's base column, each node's
        // children where its column info points.
        int c = pv.tree_base[p];
        for (int level = 0; level < L; ++level) {
          const float a = row[c] + bias_s[c];
          out[level] = a;
          if (level < D) {
            const uint32_t info = info_s[c];
            int r = go_right(a);
            if (!((info >> (18 + r)) & 1)) r ^= 1;  // pruned child: its sibling
            n = 2 * n + 1 + r;
            c = (info >> (9 * r)) & 511;
          }
        }
      }
      rec_next[static_cast<int64_t>(p) * T + t] = n;
    }
    __syncthreads();
  }
}

template <class C>
constexpr size_t top_lds_bytes() {
  // Main-loop stages, or the epilogue's logits plus its per-column arrays.
  constexpr size_t epi = size_t(C::WM) * (C::BN + 4) * 4 + size_t(C::BN) * 8;
  return C::kLdsBytes > epi ? C::kLdsBytes : epi;
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void route_top_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, const uint16_t* __restrict__ b,
    float* __restrict__ rec_logit, int32_t* __restrict__ rec_next, int T, int d, int P, int D,
    int L, int stride, int64_t N, int tiles_n, PruneView pv) {
  extern __shared__ __align__(16) uint16_t smem[];
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int tn = logical % tiles_n;
  const int tm = logical / tiles_n;
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;
  XLoader<C> la;
  la.x = x;
  la.d = d;
  la.T = T;
  la.m0 = m0;
  la.tid = threadIdx.x;
  NodeRowLoader<C> lb;
  lb.W = W;
  lb.packed = pv.W_packed;
  lb.d = d;
  lb.P = P;
  lb.L = L;
  lb.n0 = n0;
  lb.tid = threadIdx.x;
  lb.N = N;
  const ColMeta cm = load_col_meta<C>(b, P, L, N, n0, pv);
  f32x16_t acc[C::kTm][C::kTn];
  gemm_mainloop<C>(acc, smem, d, la, lb);
  top_walk_epilogue<C>(acc, reinterpret_cast<float*>(smem), cm, rec_logit, rec_next, T, P, D, L,
                       stride, N, m0, n0, pv);
}

// Same product through the direct-to-LDS multi-stage main loop.
template <class C>
__global__ __launch_bounds__(C::kThreads) void route_top_direct_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, const uint16_t* __restrict__ b,
    float* __restrict__ rec_logit, int32_t* __restrict__ rec_next, int T, int d, int P, int D,
    int L, int stride, int64_t N, int tiles_n, PruneView pv) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int tn = logical % tiles_n;
  const int tm = logical / tiles_n;
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;
  const int cmask = (1 << L) - 1;
  auto a_row = [&](int i) {
    const int r = m0 + i < T ? m0 + i : T - 1;
    return x + static_cast<size_t>(r) * d;
  };
  auto b_row = [&](int j) {
    if (pv.W_packed) return pv.W_packed + static_cast<int64_t>(n0 + j) * d;
    const int gc = n0 + j;
    const int p = gc >> L;
    const int n = gc & cmask;
    const bool used = p < P && n < cmask;
    return W + (used ? (static_cast<int64_t>(p) * N + n) * d : 0);
  };
  const ColMeta cm = load_col_meta<C>(b, P, L, N, n0, pv);
  f32x16_t acc[C::kTm][C::kTn];
  gemm_mainloop_direct<C>(acc, lds, d, a_row, b_row);
  top_walk_epilogue<C>(acc, reinterpret_cast<float*>(lds), cm, rec_logit, rec_next, T, P, D, L,
                       stride, N, m0, n0, pv);
}

// The same product split in two halves of K, for shapes whose few column
// tiles leave too few token tiles to fill the chip (the top three levels of
// 32 trees are one 256-column tile): each workgroup reads half of x's row
// tile and half of the node rows, so the node rows, which every token tile
// needs, are streamed from L2 half as often per workgroup.  No walk here:
// the raw fp32 logits of each half go to part[(half * ncols + col) * T + t]
// (token-fastest, ncols = tiles_n * BN), and the token-tile kernel that
// takes the deep levels sums the halves, adds the bias and walks.  Logical
// tiles are half-major, so the workgroups of one XCD share one half of the
// node rows in its L2.
template <class C>
__global__ __launch_bounds__(C::kThreads) void route_top_part_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, float* __restrict__ part,
    int T, int d, int P, int L, int64_t N, int tiles_m, int tiles_n) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int per = tiles_m * tiles_n;
  const int half = logical / per;
  const int rem = logical - half * per;
  const int tn = rem % tiles_n;
  const int tm = rem / tiles_n;
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;
  const int cmask = (1 << L) - 1;
  const int kh = d / 2;
  const int64_t k0 = static_cast<int64_t>(half) * kh;
  auto a_row = [&](int i) {
    const int r = m0 + i < T ? m0 + i : T - 1;
    return x + static_cast<size_t>(r) * d + k0;
  };
  auto b_row = [&](int j) {
    const int gc = n0 + j;
    const int p = gc >> L;
    const int n = gc & cmask;
    const bool used = p < P && n < cmask;
    return W + (used ? (static_cast<int64_t>(p) * N + n) * d : 0) + k0;
  };
  f32x16_t acc[C::kTm][C::kTn];
  gemm_mainloop_direct<C>(acc, lds, kh, a_row, b_row);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = wave / C::kWavesN;
  const int wn = wave % C::kWavesN;
  const int ncols = tiles_n * C::BN;
  float* out = part + static_cast<int64_t>(half) * ncols * T;
  // Lane l holds token row (block row + l % 32) and columns
  // 8 (r / 4) + 4 (l / 32) + r % 4: a store instruction writes 32
  // consecutive tokens of two columns.
#pragma unroll
  for (int i = 0; i < C::kTm; ++i) {
    const int t = m0 + wm * C::WM + i * 32 + (lane & 31);
    if (t < T) {
#pragma unroll
      for (int j = 0; j < C::kTn; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int col = n0 + wn * C::WN + j * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
          out[static_cast<int64_t>(col) * T + t] = acc[i][j][r];
        }
    }
  }
}

// H for fully routed paths (L = D+1).  One workgroup per (tile of kHbTok
// tokens, tree p): the tree's v rows are staged in LDS once (widened to fp32
// when they fit in 32 KB, else kept bf16) and reused by every token of the
// tile (the top levels' rows are shared by all of them); the tile's GELU(a)
// values and leaves come from the routing records.  Each thread then forms
// 16 outputs, 8 in each half of the token's row, of
//     H[t, p*h : (p+1)*h] = sum over l of GELU(a_l) * V_node[p, n_l, :]
// (GELU before the sum: explainer section 3.C) as two 16-byte stores; the
// h/16 threads of a token read consecutive 16-byte pieces of each staged
// half row and write its 2h-byte segment.  The depth and the chunk count per
// token are template parameters (all per-level reads issue together; index
// math is shifts).  kHbThreads = 2 kHbTok threads share the tile's tokens:
// the LDS of a tile (about 40 KB at h = 128) allows four workgroups per
// compute unit, and twice the tile's token count in threads keeps eight
// waves per SIMD in flight.
constexpr int kHbTok = 256;
constexpr int kHbThreads = 512;

// Eight consecutive V values of row-major staged rows (fp32 or bf16).
template <bool F32>
__device__ __forceinline__ void load_v8(const unsigned char* vs, size_t elem, float* v) {
  if constexpr (F32) {
    const float4* src = reinterpret_cast<const float4*>(vs + elem * 4);
    const float4 f0 = src[0], f1 = src[1];
    v[0] = f0.x; v[1] = f0.y; v[2] = f0.z; v[3] = f0.w;
    v[4] = f1.x; v[5] = f1.y; v[6] = f1.z; v[7] = f1.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(vs + elem * 2);
    v[0] = bf16lo(u.x); v[1] = bf16hi(u.x); v[2] = bf16lo(u.y); v[3] = bf16hi(u.y);
    v[4] = bf16lo(u.z); v[5] = bf16hi(u.z); v[6] = bf16lo(u.w); v[7] = bf16hi(u.w);
  }
}

template <int LEVELS, int HSHIFT, bool F32>
__global__ __launch_bounds__(kHbThreads) void hbuild_kernel(const float* __restrict__ rec_logit,
                                                     const int32_t* __restrict__ rec_next,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ H,
                                                     int32_t* __restrict__ path_out, int T, int P,
                                                     int64_t N, int post, int blocked) {
  constexpr int L = LEVELS;
  constexpr int D = LEVELS - 1;
  constexpr int h = 16 << HSHIFT;     // node output width
  constexpr int kChunks = 1 << HSHIFT;  // 16-output chunks per token
  constexpr int kEsz = F32 ? 4 : 2;
  extern __shared__ __align__(16) unsigned char hb_lds[];
  // Workgroups launched together cover all trees of the same token block,
  // so the stores in flight fill whole rows of H, and workgroup b runs on
  // XCD b % 8, which then stages only its own trees' V rows.
  const int p = static_cast<int>(blockIdx.x % static_cast<unsigned>(P));
  const int t0 = static_cast<int>(blockIdx.x / static_cast<unsigned>(P)) * kHbTok;
  const int ntok = min(kHbTok, T - t0);
  unsigned char* vs = hb_lds;                                               // N x h
  float* gl = reinterpret_cast<float*>(hb_lds + size_t(N) * h * kEsz);     // kHbTok x L
  int32_t* leaf = reinterpret_cast<int32_t*>(gl + kHbTok * L);             // kHbTok
  static_assert(kHbTok % kHbThreads == 0 || kHbThreads % kHbTok == 0, "token loop");
  const uint16_t* Vp = V + static_cast<int64_t>(p) * N * h;
  // Every load of the staging phase is issued before any is waited for (a
  // loop of load, wait and store would cost one memory round trip per
  // iteration).
  if constexpr (F32) {
    // Small trees (N * h * 4 <= 32 KB: at most 1024 16-byte pieces),
    // widened to fp32.
    constexpr int kPer = 1024 / kHbThreads;
    const int pieces = static_cast<int>(N) * (h / 8);
    uint4 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * kHbThreads;
      v[u] = ldg16(Vp + static_cast<size_t>(e < pieces ? e : 0) * 8);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * kHbThreads;
      if (e < pieces) {
        float4* dst = reinterpret_cast<float4*>(vs + static_cast<size_t>(e) * 32);
        dst[0] = make_float4(bf16lo(v[u].x), bf16hi(v[u].x), bf16lo(v[u].y), bf16hi(v[u].y));
        dst[1] = make_float4(bf16lo(v[u].z), bf16hi(v[u].z), bf16lo(v[u].w), bf16hi(v[u].w));
      }
    }
  } else {
    // The tree's V rows are contiguous: copied straight into LDS, 1 KB per
    // wave-wide load (lane i at byte 16 i).
    const unsigned char* src = reinterpret_cast<const unsigned char*>(Vp);
    const int total = static_cast<int>(N) * h * 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    for (int base = wave * 1024; base < total; base += (kHbThreads / kWave) * 1024)
      if (base + lane * 16 < total)
        __builtin_amdgcn_global_load_lds(src + base + lane * 16, vs + base, 16, 0, 0);
  }
  // Per-node weights of the V rows: GELU(a) per node, or a itself when GELU is
  // applied to the summed vector instead.
  const float* rl = rec_logit + (static_cast<int64_t>(p) * T + t0) * L;
  constexpr int kRec = (kHbTok * L + kHbThreads - 1) / kHbThreads;
  float lv[kRec];
#pragma unroll
  for (int u = 0; u < kRec; ++u) {
    const int i = threadIdx.x + u * kHbThreads;
    lv[u] = rl[i < ntok * L ? i : 0];
  }
  constexpr int kLeafPer = (kHbTok + kHbThreads - 1) / kHbThreads;
  int32_t nl[kLeafPer];
#pragma unroll
  for (int u = 0; u < kLeafPer; ++u) {
    const int i = threadIdx.x + u * kHbThreads;
    nl[u] = rec_next[static_cast<int64_t>(p) * T + t0 + (i < ntok ? i : 0)];
  }
#pragma unroll
  for (int u = 0; u < kRec; ++u) {
    const int i = threadIdx.x + u * kHbThreads;
    if (i < ntok * L) gl[i] = post ? lv[u] : gelu_tanh(lv[u]);
  }
#pragma unroll
  for (int u = 0; u < kLeafPer; ++u) {
    const int i = threadIdx.x + u * kHbThreads;
    if (i < ntok) {
      leaf[i] = nl[u];
      if (path_out) path_out[static_cast<int64_t>(t0 + i) * P + p] = nl[u] - ((1 << D) - 1);
    }
  }
  wait_vmcnt<0>();  // the copies into LDS have landed
  __syncthreads();
  uint16_t* Hp = H + static_cast<int64_t>(p) * h;
  for (int e = threadIdx.x; e < (ntok << HSHIFT); e += blockDim.x) {
    const int i = e >> HSHIFT;
    // Columns ja..ja+7 and jb..jb+7: the lanes of a token read consecutive
    // pieces of each half row (no LDS bank conflicts), and write them.
    const int ja = (e & (kChunks - 1)) * 8;
    const int jb = h / 2 + ja;
    const int32_t lf = leaf[i];
    const float* g = gl + i * L;
    float acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int n = ((lf + 1) >> (D - l)) - 1;  // ancestor of the leaf at level l
      float v[16];
      load_v8<F32>(vs, static_cast<size_t>(n) * h + ja, v);
      load_v8<F32>(vs, static_cast<size_t>(n) * h + jb, v + 8);
      const float gg = g[l];
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] += gg * v[q];
    }
    if (post) {
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = gelu_tanh(acc[q]);
    }
    uint16_t* pa;
    uint16_t* pb;
    if (blocked) {  // element (t, k) at ((k / 32) * T + t) * 32 + k % 32
      const int64_t ka = static_cast<int64_t>(p) * h + ja, kb = ka + h / 2;
      const int64_t tt = static_cast<int64_t>(t0 + i) * 32;
      pa = H + (ka >> 5) * (static_cast<int64_t>(T) << 5) + tt + (ka & 31);
      pb = H + (kb >> 5) * (static_cast<int64_t>(T) << 5) + tt + (kb & 31);
    } else {
      uint16_t* row = Hp + static_cast<int64_t>(t0 + i) * P * h;
      pa = row + ja;
      pb = row + jb;
    }
    *reinterpret_cast<uint4*>(pa) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    *reinterpret_cast<uint4*>(pb) =
        make_uint4(pack_bf16x2(acc[8], acc[9]), pack_bf16x2(acc[10], acc[11]),
                   pack_bf16x2(acc[12], acc[13]), pack_bf16x2(acc[14], acc[15]));
  }
}

bool hbuild_f32(const Dims& s) { return size_t(s.N) * s.h * 4 <= 32 * 1024; }

size_t hbuild_lds_bytes(const Dims& s) {
  return size_t(s.N) * s.h * (hbuild_f32(s) ? 4 : 2) + size_t(kHbTok) * (s.D + 1) * 4 +
         kHbTok * 4;
}

// Column tiles of the dense product over levels < L: whole trees of 2^L
// columns, or the pruning table's packed tiles.
int top_col_tiles(const Dims& s, int L) {
  if (s.prune) return s.prune->col_tiles;
  return static_cast<int>(((static_cast<int64_t>(s.P) << L) + 255) / 256);
}

template <class C, bool kDirect>
hipError_t launch_top_cfg(const Dims& s, int L, int stride, const void* x, const void* W,
                          const void* b, float* rec_logit, int32_t* rec_next, hipStream_t st) {
  const int tiles_m = static_cast<int>((s.T + C::BM - 1) / C::BM);
  const int tiles_n = top_col_tiles(s, L);
  const PruneView pv = s.prune ? *s.prune : PruneView{};
  void (*kern)(const uint16_t*, const uint16_t*, const uint16_t*, float*, int32_t*, int, int, int,
               int, int, int, int64_t, int, PruneView);
  if constexpr (kDirect)
    kern = route_top_direct_kernel<C>;
  else
    kern = route_top_kernel<C>;
  const size_t lds = top_lds_bytes<C>();
  {
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void*>(kern), static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  kern<<<dim3(tiles_m * tiles_n), dim3(C::kThreads), lds, st>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W),
      static_cast<const uint16_t*>(b), rec_logit, rec_next, static_cast<int>(s.T), s.d, s.P, s.D,
      L, stride, s.N, tiles_n, pv);
  return hipGetLastError();
}

using MidTile = TileCfg<128, 256, 64, 64, 128>;
using SmallTile = TileCfg<64, 256, 64, 64, 64>;
using TopDirect = DirectCfg<256, 256, 128, 64, 4>;
// 64 tokens x 256 columns on four waves: 80 KB of stages, so two
// workgroups share a compute unit; for few column tiles (the top three
// levels of 32 trees are one tile) it fills the chip where 256-token tiles
// would leave most compute units idle.
using TopDirect64 = DirectCfg<64, 256, 64, 64, 4>;
// 128 tokens x 256 columns on eight waves (96 KB of stages).
using TopDirect128 = DirectCfg<128, 256, 64, 64, 4>;


// One workgroup per packed row: packed[i] = W row colmap[i] (zeros for -1).
__global__ __launch_bounds__(256) void prune_pack_kernel(const uint16_t* __restrict__ W,
                                                         const int32_t* __restrict__ colmap,
                                                         uint16_t* __restrict__ packed, int d) {
  const int i = blockIdx.x;
  const int64_t src = colmap[i];
  uint16_t* dst = packed + static_cast<int64_t>(i) * d;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    const uint4 v = src >= 0 ? ldg16(W + src * d + c) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(dst + c) = v;
  }
}

}  // namespace

hipError_t launch_prune_pack(const void* W, const int32_t* colmap, void* packed, int rows, int d,
                             hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  prune_pack_kernel<<<dim3(rows), dim3(256), 0, st>>>(static_cast<const uint16_t*>(W), colmap,
                                                      static_cast<uint16_t*>(packed), d);
  return hipGetLastError();
}

// The split form is taken for unpruned token-tile plans (the deep kernel
// walks the top levels) when 128-token tiles alone give fewer than 256
// workgroups and the two K halves at least 256.
bool route_top_split_wanted(const Dims& s, int L) {
  if (s.prune || s.dtype != 1 || s.d % 64 != 0 || (1 << L) > TopDirect128::BN) return false;
  const int64_t tiles = (s.T + TopDirect128::BM - 1) / TopDirect128::BM * top_col_tiles(s, L);
  return tiles < 256 && 2 * tiles >= 256;
}

size_t route_top_split_bytes(const Dims& s, int L) {
  return size_t(2) * size_t(top_col_tiles(s, L)) * TopDirect128::BN * size_t(s.T) * 4;
}

int route_top_split_cols(const Dims& s, int L) { return top_col_tiles(s, L) * TopDirect128::BN; }

hipError_t launch_route_top_split(const Dims& s, int L, const void* x, const void* W,
                                  float* part, hipStream_t st) {
  using C = TopDirect128;
  const int tiles_m = static_cast<int>((s.T + C::BM - 1) / C::BM);
  const int tiles_n = top_col_tiles(s, L);
  auto kern = route_top_part_kernel<C>;
  {
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void*>(kern), static_cast<int>(C::kLdsBytes));
    if (e != hipSuccess) return e;
  }
  kern<<<dim3(2 * tiles_m * tiles_n), dim3(C::kThreads), C::kLdsBytes, st>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), part,
      static_cast<int>(s.T), s.d, s.P, L, s.N, tiles_m, tiles_n);
  return hipGetLastError();
}

bool route_top_supported(const Dims& s, int L) {
  return s.dtype == 1 && s.d % TopTile::BK == 0 && s.h % 8 == 0 && L >= 1 && L <= s.D + 1 &&
         (1 << L) <= TopTile::BN && (L <= s.D || hbuild_supported(s));
}

hipError_t launch_route_top(const Dims& s, int L, int stride, const void* x, const void* W,
                            const void* b, float* rec_logit, int32_t* rec_next, hipStream_t st) {
  if (stride < L) return hipErrorInvalidValue;
  // A pruning table packs the rows of one split level only.
  if (s.prune && s.prune->L != L) return hipErrorInvalidValue;
  // Enough tiles to cover the 256 compute units: shrink the token tile when
  // the column count is small (few trees or few levels).
  const int64_t tiles_n = top_col_tiles(s, L);
  // Direct-to-LDS tiles of 256, 128 or 64 tokens (each at least 256 tiles):
  // the one whose busiest compute unit has the least output area (tiles per
  // unit x tile area), ties to the larger tile.
  int64_t best = INT64_MAX;
  int pick = 0;
  for (int bm : {256, 128, 64}) {
    const int64_t tiles = (s.T + bm - 1) / bm * tiles_n;
    const int64_t area = (tiles + 255) / 256 * bm;
    if ((1 << L) <= TopDirect::BN && tiles >= 256 && area < best) {
      best = area;
      pick = bm;
    }
  }
  if (pick == 256)
    return launch_top_cfg<TopDirect, true>(s, L, stride, x, W, b, rec_logit, rec_next, st);
  if (pick == 128)
    return launch_top_cfg<TopDirect128, true>(s, L, stride, x, W, b, rec_logit, rec_next, st);
  if (pick == 64)
    return launch_top_cfg<TopDirect64, true>(s, L, stride, x, W, b, rec_logit, rec_next, st);
  if (((s.T + 127) / 128) * tiles_n >= 256)
    return launch_top_cfg<MidTile, false>(s, L, stride, x, W, b, rec_logit, rec_next, st);
  return launch_top_cfg<SmallTile, false>(s, L, stride, x, W, b, rec_logit, rec_next, st);
}

namespace {
template <int LEVELS, int HSHIFT, bool F32>
hipError_t launch_hbuild_l(const Dims& s, const float* rec_logit, const int32_t* rec_next,
                           const void* V, void* H, int32_t* path_out, bool blocked,
                           hipStream_t st) {
  const size_t lds = hbuild_lds_bytes(s);
  auto kern = hbuild_kernel<LEVELS, HSHIFT, F32>;
  {
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void*>(kern), 160 * 1024);
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = (s.T + kHbTok - 1) / kHbTok * s.P;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  kern<<<dim3(static_cast<unsigned>(blocks)), dim3(kHbThreads), lds, st>>>(rec_logit, rec_next, static_cast<const uint16_t*>(V),
                                     static_cast<uint16_t*>(H), path_out, static_cast<int>(s.T),
                                     s.P, s.N, s.variant, blocked ? 1 : 0);
  return hipGetLastError();
}

template <int LEVELS, int HSHIFT>
hipError_t launch_hbuild_h(const Dims& s, const float* rec_logit, const int32_t* rec_next,
                           const void* V, void* H, int32_t* path_out, bool blocked,
                           hipStream_t st) {
  if (hbuild_f32(s))
    return launch_hbuild_l<LEVELS, HSHIFT, true>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
  return launch_hbuild_l<LEVELS, HSHIFT, false>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
}

template <int LEVELS>
hipError_t launch_hbuild_d(const Dims& s, const float* rec_logit, const int32_t* rec_next,
                           const void* V, void* H, int32_t* path_out, bool blocked,
                           hipStream_t st) {
  switch (s.h) {
    case 64: return launch_hbuild_h<LEVELS, 2>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 128: return launch_hbuild_h<LEVELS, 3>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 256: return launch_hbuild_h<LEVELS, 4>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 512: return launch_hbuild_h<LEVELS, 5>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    default: return hipErrorInvalidValue;  // hbuild_supported() excludes other widths
  }
}
}  // namespace

bool hbuild_supported(const Dims& s) {
  return s.D + 1 <= 8 && (s.h == 64 || s.h == 128 || s.h == 256 || s.h == 512) &&
         hbuild_lds_bytes(s) <= 160 * 1024;
}

hipError_t launch_hbuild(const Dims& s, const float* rec_logit, const int32_t* rec_next,
                         const void* V, void* H, int32_t* path_out, bool blocked,
                         hipStream_t st) {
  switch (s.D + 1) {
    case 1: return launch_hbuild_d<1>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 2: return launch_hbuild_d<2>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 3: return launch_hbuild_d<3>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 4: return launch_hbuild_d<4>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 5: return launch_hbuild_d<5>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 6: return launch_hbuild_d<6>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 7: return launch_hbuild_d<7>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    case 8: return launch_hbuild_d<8>(s, rec_logit, rec_next, V, H, path_out, blocked, st);
    default: return hipErrorInvalidValue;  // the dense path covers D+1 <= 8 only
  }
}

}  // namespace fff
