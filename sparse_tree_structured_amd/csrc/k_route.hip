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
  int d, P, L, n0, tid;
  int64_t N;
  __device__ __forceinline__ void load(int k0) {
    rl.load([&](int i) {
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
// LDS of at least WM * (BN + 4) floats, free for reuse.
template <class C>
__device__ __forceinline__ void top_walk_epilogue(const f32x16_t (&acc)[C::kTm][C::kTn], float* lg,
                                                  const uint16_t* __restrict__ b,
                                                  float* __restrict__ rec_logit,
                                                  int32_t* __restrict__ rec_next, int T, int P,
                                                  int D, int L, int64_t N, int m0, int n0) {
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
  const int tpt = C::BN >> L;  // trees per tile
  const int p_base = n0 >> L;
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
      const float* row = lg + tr * kPitch + tp * cpt;
      const uint16_t* bp = b + static_cast<int64_t>(p) * N;
      float* out = rec_logit + (static_cast<int64_t>(p) * T + t) * L;
      int n = 0;
      for (int level = 0; level < L; ++level) {
        const float a = row[n] + bf16_to_f32(bp[n]);
        out[level] = a;
        if (level < D) n = 2 * n + 1 + go_right(a);
      }
      rec_next[static_cast<int64_t>(p) * T + t] = n;
    }
    __syncthreads();
  }
}

template <class C>
constexpr size_t top_lds_bytes() {
  return C::kLdsBytes > size_t(C::WM) * (C::BN + 4) * 4 ? C::kLdsBytes
                                                        : size_t(C::WM) * (C::BN + 4) * 4;
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void route_top_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, const uint16_t* __restrict__ b,
    float* __restrict__ rec_logit, int32_t* __restrict__ rec_next, int T, int d, int P, int D,
    int L, int64_t N, int tiles_n) {
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
  lb.d = d;
  lb.P = P;
  lb.L = L;
  lb.n0 = n0;
  lb.tid = threadIdx.x;
  lb.N = N;
  f32x16_t acc[C::kTm][C::kTn];
  gemm_mainloop<C>(acc, smem, d, la, lb);
  top_walk_epilogue<C>(acc, reinterpret_cast<float*>(smem), b, rec_logit, rec_next, T, P, D, L, N,
                       m0, n0);
}

// Same product through the direct-to-LDS multi-stage main loop.
template <class C>
__global__ __launch_bounds__(C::kThreads) void route_top_direct_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, const uint16_t* __restrict__ b,
    float* __restrict__ rec_logit, int32_t* __restrict__ rec_next, int T, int d, int P, int D,
    int L, int64_t N, int tiles_n) {
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
    const int gc = n0 + j;
    const int p = gc >> L;
    const int n = gc & cmask;
    const bool used = p < P && n < cmask;
    return W + (used ? (static_cast<int64_t>(p) * N + n) * d : 0);
  };
  f32x16_t acc[C::kTm][C::kTn];
  gemm_mainloop_direct<C>(acc, lds, d, a_row, b_row);
  top_walk_epilogue<C>(acc, reinterpret_cast<float*>(lds), b, rec_logit, rec_next, T, P, D, L, N,
                       m0, n0);
}

// H for fully routed paths (L = D+1).  One workgroup per token: first the
// P*(D+1) GELU values and node ids into LDS, then each thread forms 8
// consecutive outputs (one 16-byte store) of the token's H row.
__global__ __launch_bounds__(256) void hbuild_kernel(const float* __restrict__ rec_logit,
                                                     const int32_t* __restrict__ rec_next,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ H,
                                                     int32_t* __restrict__ path_out, int T, int P,
                                                     int D, int h, int64_t N) {
  extern __shared__ float gl[];  // [P][D+1] GELU values, then [P] leaf heap ids
  int32_t* leaf = reinterpret_cast<int32_t*>(gl + P * (D + 1));
  const int t = blockIdx.x;
  const int L = D + 1;
  for (int i = threadIdx.x; i < P * L; i += blockDim.x) {
    const int p = i / L;
    const int l = i - p * L;
    gl[i] = gelu_tanh(rec_logit[(static_cast<int64_t>(p) * T + t) * L + l]);
  }
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int32_t n = rec_next[static_cast<int64_t>(p) * T + t];
    leaf[p] = n;
    if (path_out) path_out[static_cast<int64_t>(t) * P + p] = n - ((1 << D) - 1);
  }
  __syncthreads();
  const int chunks = h / 8;
  uint16_t* Ht = H + static_cast<int64_t>(t) * P * h;
  for (int c = threadIdx.x; c < P * chunks; c += blockDim.x) {
    const int p = c / chunks;
    const int j0 = (c - p * chunks) * 8;
    const int32_t lf = leaf[p];
    const uint16_t* Vp = V + static_cast<int64_t>(p) * N * h + j0;
    float acc[8] = {};
    for (int l = 0; l < L; ++l) {
      const int64_t n = ((lf + 1) >> (D - l)) - 1;  // ancestor of the leaf at level l
      const float g = gl[p * L + l];
      const uint4 v = ldg16(Vp + n * h);
      acc[0] += g * bf16lo(v.x);
      acc[1] += g * bf16hi(v.x);
      acc[2] += g * bf16lo(v.y);
      acc[3] += g * bf16hi(v.y);
      acc[4] += g * bf16lo(v.z);
      acc[5] += g * bf16hi(v.z);
      acc[6] += g * bf16lo(v.w);
      acc[7] += g * bf16hi(v.w);
    }
    *reinterpret_cast<uint4*>(Ht + p * h + j0) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

template <class C, bool kDirect>
hipError_t launch_top_cfg(const Dims& s, int L, const void* x, const void* W, const void* b,
                          float* rec_logit, int32_t* rec_next, hipStream_t st) {
  const int tiles_m = static_cast<int>((s.T + C::BM - 1) / C::BM);
  const int64_t cols = static_cast<int64_t>(s.P) << L;
  const int tiles_n = static_cast<int>((cols + C::BN - 1) / C::BN);
  void (*kern)(const uint16_t*, const uint16_t*, const uint16_t*, float*, int32_t*, int, int, int,
               int, int, int64_t, int);
  if constexpr (kDirect)
    kern = route_top_direct_kernel<C>;
  else
    kern = route_top_kernel<C>;
  const size_t lds = top_lds_bytes<C>();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  kern<<<dim3(tiles_m * tiles_n), dim3(C::kThreads), lds, st>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W),
      static_cast<const uint16_t*>(b), rec_logit, rec_next, static_cast<int>(s.T), s.d, s.P, s.D,
      L, s.N, tiles_n);
  return hipGetLastError();
}

using MidTile = TileCfg<128, 256, 64, 64, 128>;
using SmallTile = TileCfg<64, 256, 64, 64, 64>;
using TopDirect = DirectCfg<256, 256, 128, 64, 4>;

}  // namespace

bool route_top_supported(const Dims& s, int L) {
  return s.dtype == 1 && s.d % TopTile::BK == 0 && s.h % 8 == 0 && L >= 1 && L <= s.D + 1 &&
         (1 << L) <= TopTile::BN && int64_t(s.P) * (s.D + 2) * 4 <= 65536;
}

hipError_t launch_route_top(const Dims& s, int L, const void* x, const void* W, const void* b,
                            float* rec_logit, int32_t* rec_next, hipStream_t st) {
  // Enough tiles to cover the 256 compute units: shrink the token tile when
  // the column count is small (few trees or few levels).
  const int64_t tiles_n = ((static_cast<int64_t>(s.P) << L) + TopTile::BN - 1) / TopTile::BN;
  if (((s.T + 255) / 256) * tiles_n >= 256)
    return launch_top_cfg<TopDirect, true>(s, L, x, W, b, rec_logit, rec_next, st);
  if (((s.T + 127) / 128) * tiles_n >= 256)
    return launch_top_cfg<MidTile, false>(s, L, x, W, b, rec_logit, rec_next, st);
  return launch_top_cfg<SmallTile, false>(s, L, x, W, b, rec_logit, rec_next, st);
}

hipError_t launch_hbuild(const Dims& s, const float* rec_logit, const int32_t* rec_next,
                         const void* V, void* H, int32_t* path_out, hipStream_t st) {
  const size_t lds = static_cast<size_t>(s.P) * (s.D + 1) * sizeof(float) + s.P * sizeof(int32_t);
  hbuild_kernel<<<dim3(static_cast<unsigned>(s.T)), dim3(256), lds, st>>>(
      rec_logit, rec_next, static_cast<const uint16_t*>(V), static_cast<uint16_t*>(H), path_out,
      static_cast<int>(s.T), s.P, s.D, s.h, s.N);
  return hipGetLastError();
}

}  // namespace fff
