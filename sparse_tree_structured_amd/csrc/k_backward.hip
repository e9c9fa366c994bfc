// Backward pass of the FFF layer on gfx950: gradients of sum(y * dy) with
// the forward's paths held fixed.
//
// The explainer page ("Dynamic sparsity in tree-structured feed-forward
// layers at scale", gist.science, section 3.B) describes gradients that
// reach only the nodes a token visits; the hard decision itself has no
// gradient (the pages name no estimator).  Per token t, tree p and visited
// node n (logit a, level l), with dH = dy . W_out^T:
//   FFF      da = GELU'(a) * (dH_p . v_n),        dV_n += GELU(a) * dH_p
//   FFF-post s = sum over the path of a * v_n,    ds = GELU'(s) (*) dH_p,
//            da = ds . v_n,                       dV_n += a * ds
//   db_n += da,  dW_n += da * x_t,  dx_t += da * w_n,  dW_out = H^T . dy.
//
// Generic kernels (any shape, fp32 or bf16): one wavefront per (token,
// tree) and fp32 atomics for the sums over tokens.
//
// Matrix-core path (bf16, every level dense, as the forward's default
// plan): the sums over tokens and nodes are products with the masked
// matrix DA[t, (p, n)] (da at the token's visited nodes, 0 elsewhere, one
// column per node of the dense levels), the same masked form the forward
// uses for the logits (explainer page, section 2, Implementation):
//   dH   = dy . W_out^T             dx     = DA . W_top
//   dW   = DA^T . x                 dW_out = H^T . dy
//   dV_p = G_p^T . dS_p  (G: GELU(a), or a for FFF-post, at visited nodes;
//                         dS_p: dH_p, or GELU'(s) * dH_p)
// all as one bf16 "A . B^T" kernel over K-contiguous rows (the forward's
// direct-to-LDS main loop), with the token-major operands transposed once.
#include <algorithm>

#include "fff.h"

#include "common.hpp"
#include "launch.hpp"
#include "mfma_tile.hpp"

namespace fff {
namespace {

// GELU' of the tanh form: 0.5 (1 + tanh u) + 0.5 a (1 - tanh^2 u) u'(a),
// u = sqrt(2/pi) (a + 0.044715 a^3).
__device__ __forceinline__ float gelu_tanh_grad(float a) {
  const float k0 = 0.7978845608028654f;
  const float k1 = 0.044715f;
  const float th = tanhf(k0 * (a + k1 * a * a * a));
  return 0.5f * (1.0f + th) + 0.5f * a * (1.0f - th * th) * k0 * (1.0f + 3.0f * k1 * a * a);
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0.0f;
}

// dH[t,k] = sum_c dy[t,c] W_out[k,c]  (fp32).
template <typename E>
__global__ __launch_bounds__(256) void bwd_dh_generic_kernel(const E* __restrict__ dy,
                                                             const E* __restrict__ Wout,
                                                             float* __restrict__ dH, int64_t T,
                                                             int d, int64_t K) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < T * K;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = e / K;
    const int64_t k = e - t * K;
    float acc = 0.0f;
    for (int c = 0; c < d; ++c) acc += Elem<E>::ld(dy, t * d + c) * Elem<E>::ld(Wout, k * d + c);
    dH[e] = acc;
  }
}

// H[t, p*h + j] in fp32 from the routing records (both variants).
template <typename E>
__global__ __launch_bounds__(256) void bwd_h_generic_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ leaf_ws, const E* __restrict__ V,
    float* __restrict__ H, int64_t T, int P, int D, int h, int64_t N, int post) {
  const int64_t K = static_cast<int64_t>(P) * h;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < T * K;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = e / K;
    const int64_t col = e - t * K;
    const int p = static_cast<int>(col / h);
    const int j = static_cast<int>(col - static_cast<int64_t>(p) * h);
    const int64_t pair = t * P + p;
    const int32_t leaf = leaf_ws[pair];
    const E* Vp = V + static_cast<int64_t>(p) * N * h;
    float acc = 0.0f;
    int64_t n = 0;
    for (int level = 0; level <= D; ++level) {
      const float a = logits[pair * (D + 1) + level];
      acc += (post ? a : gelu_tanh(a)) * Elem<E>::ld(Vp, n * h + j);
      if (level < D) n = 2 * n + 1 + ((leaf >> (D - 1 - level)) & 1);
    }
    H[e] = post ? gelu_tanh(acc) : acc;
  }
}

// One wavefront per (token, tree): the path's da, and the atomic sums of
// db, dW, dV and the fp32 dx accumulator.
template <typename E>
__global__ __launch_bounds__(256) void bwd_paths_generic_kernel(
    const E* __restrict__ x, const E* __restrict__ W, const E* __restrict__ V,
    const float* __restrict__ logits, const int32_t* __restrict__ leaf_ws,
    const float* __restrict__ dH, float* __restrict__ dW, float* __restrict__ db,
    float* __restrict__ dV, float* __restrict__ dxacc, int64_t T, int d, int P, int D, int h,
    int64_t N, int post) {
  constexpr int kMaxL = FFF_MAX_DEPTH + 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (pair >= T * P) return;  // whole wavefront leaves together
  const int64_t t = pair / P;
  const int p = static_cast<int>(pair % P);
  const int L = D + 1;
  const int32_t leaf = leaf_ws[pair];
  int64_t node[kMaxL];
  float a[kMaxL], g[kMaxL];
  int64_t n = 0;
  for (int l = 0; l < L; ++l) {
    node[l] = n;
    a[l] = logits[pair * L + l];
    g[l] = 0.0f;
    if (l < D) n = 2 * n + 1 + ((leaf >> (D - 1 - l)) & 1);
  }
  const E* Vp = V + static_cast<int64_t>(p) * N * h;
  float* dVp = dV + static_cast<int64_t>(p) * N * h;
  const float* dHt = dH + t * P * h + static_cast<int64_t>(p) * h;
  for (int j = lane; j < h; j += kWave) {
    float dj = dHt[j];
    if (post) {
      float s = 0.0f;
      for (int l = 0; l < L; ++l) s += a[l] * Elem<E>::ld(Vp, node[l] * h + j);
      dj *= gelu_tanh_grad(s);
    }
    for (int l = 0; l < L; ++l) {
      g[l] += dj * Elem<E>::ld(Vp, node[l] * h + j);
      atomicAdd(dVp + node[l] * h + j, (post ? a[l] : gelu_tanh(a[l])) * dj);
    }
  }
  const E* xt = x + t * d;
  const E* Wp = W + static_cast<int64_t>(p) * N * d;
  float* dWp = dW + static_cast<int64_t>(p) * N * d;
  for (int l = 0; l < L; ++l) {
    const float gl = wave_sum(g[l]);
    const float da = post ? gl : gl * gelu_tanh_grad(a[l]);
    if (lane == 0) atomicAdd(db + static_cast<int64_t>(p) * N + node[l], da);
    for (int i = lane; i < d; i += kWave) {
      atomicAdd(dWp + node[l] * d + i, da * Elem<E>::ld(xt, i));
      atomicAdd(dxacc + t * d + i, da * Elem<E>::ld(Wp, node[l] * d + i));
    }
  }
}

// dW_out[k,c] = sum_t H[t,k] dy[t,c].
template <typename E>
__global__ __launch_bounds__(256) void bwd_dwout_generic_kernel(const float* __restrict__ H,
                                                                const E* __restrict__ dy,
                                                                float* __restrict__ dWout,
                                                                int64_t T, int d, int64_t K) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < K * d;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t k = e / d;
    const int64_t c = e - k * d;
    float acc = 0.0f;
    for (int64_t t = 0; t < T; ++t) acc += H[t * K + k] * Elem<E>::ld(dy, t * d + c);
    dWout[e] = acc;
  }
}

template <typename E>
__global__ __launch_bounds__(256) void store_dx_kernel(const float* __restrict__ acc,
                                                       E* __restrict__ dx, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    Elem<E>::st(dx, i, acc[i]);
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  return static_cast<unsigned>(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

template <typename E>
hipError_t backward_generic_t(const Dims& s, const void* x, const void* W, const void* V,
                              const void* Wout, const void* dy, void* dx, float* dW, float* db,
                              float* dV, float* dWout, const float* logits,
                              const int32_t* leaf, float* dH, float* Hf, float* dxacc,
                              hipStream_t st) {
  const int64_t nW = int64_t(s.P) * s.N * s.d, nb = int64_t(s.P) * s.N;
  const int64_t nV = int64_t(s.P) * s.N * s.h, nx = s.T * s.d, nTK = s.T * s.K;
  fill_f32_kernel<<<grid_for(nW), 256, 0, st>>>(dW, nW);
  fill_f32_kernel<<<grid_for(nb), 256, 0, st>>>(db, nb);
  fill_f32_kernel<<<grid_for(nV), 256, 0, st>>>(dV, nV);
  fill_f32_kernel<<<grid_for(nx), 256, 0, st>>>(dxacc, nx);
  bwd_dh_generic_kernel<E><<<grid_for(nTK), 256, 0, st>>>(
      static_cast<const E*>(dy), static_cast<const E*>(Wout), dH, s.T, s.d, s.K);
  bwd_h_generic_kernel<E><<<grid_for(nTK), 256, 0, st>>>(logits, leaf, static_cast<const E*>(V),
                                                          Hf, s.T, s.P, s.D, s.h, s.N, s.variant);
  const int64_t pairs = s.T * s.P;
  bwd_paths_generic_kernel<E><<<static_cast<unsigned>((pairs + 3) / 4), 256, 0, st>>>(
      static_cast<const E*>(x), static_cast<const E*>(W), static_cast<const E*>(V), logits, leaf,
      dH, dW, db, dV, dxacc, s.T, s.d, s.P, s.D, s.h, s.N, s.variant);
  bwd_dwout_generic_kernel<E><<<grid_for(s.K * s.d), 256, 0, st>>>(
      Hf, static_cast<const E*>(dy), dWout, s.T, s.d, s.K);
  store_dx_kernel<E><<<grid_for(nx), 256, 0, st>>>(dxacc, static_cast<E*>(dx), nx);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Matrix-core path.

using BwdTile = DirectCfg<256, 256, 128, 64, 4>;
// One tree's dV product is 2^L x h (128 x 128 at the headline): a quarter of
// a 256 x 256 tile, so it takes 128 x 128 tiles on 4 waves.
using BwdSmallTile = DirectCfg<128, 128, 64, 64, 4>;

// C = A . B^T over K-contiguous bf16 rows.  Grid: batches x ksplit x
// tiles, XCD-aware.  Output modes: kBf16 stores; kF32 stores, split ks of
// the k dimension writing its partial product at C + ks * split_stride (a
// separate pass sums the splits: float32 atomics here measured 0.85 ms
// slower per backward call at the OPT-1.3B shape), with rows remapped from
// the dense node layout (row r = p * 2^L + n -> p * Nn + n, the spare column
// n = 2^L - 1 dropped) when L > 0.
struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int64_t lda, ldb, ldc;
  int64_t a_bstride, b_bstride, c_bstride;  // rows per batch
  int M, N, Kk;                             // Kk: k extent of one split
  int tiles_m, tiles_n, ksplit;
  int L;
  int64_t Nn;
  int64_t split_stride;  // elements of C between the splits' partial products
};

enum GemmOut { kBf16 = 0, kF32 = 1 };

template <class C, int kOut>
__global__ __launch_bounds__(C::kThreads) void gemm_nt_kernel(GemmArgs g) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int per = g.tiles_m * g.tiles_n;
  const int tile = logical % per;
  const int rest = logical / per;
  const int ks = rest % g.ksplit;
  const int batch = rest / g.ksplit;
  const int m0 = (tile / g.tiles_n) * C::BM;
  const int n0 = (tile % g.tiles_n) * C::BN;
  const int64_t koff = static_cast<int64_t>(ks) * g.Kk;
  auto a_row = [&](int i) {
    const int r = m0 + i < g.M ? m0 + i : g.M - 1;
    return g.A + (batch * g.a_bstride + r) * g.lda + koff;
  };
  auto b_row = [&](int j) {
    const int c = n0 + j < g.N ? n0 + j : g.N - 1;
    return g.B + (batch * g.b_bstride + c) * g.ldb + koff;
  };
  f32x16_t acc[C::kTm][C::kTn];
  gemm_mainloop_direct<C>(acc, lds, g.Kk, a_row, b_row);

  // Lane holds row (m-block i, lane % 32) and, for q = 0..3, the four
  // consecutive columns 8q + 4 (lane / 32) + 0..3 of n-block j.
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = wave / C::kWavesN;
  const int wn = wave % C::kWavesN;
  const int mask = (1 << g.L) - 1;
#pragma unroll
  for (int i = 0; i < C::kTm; ++i) {
    const int row = m0 + wm * C::WM + i * 32 + (lane & 31);
    if (row >= g.M) continue;
    int64_t out_row = batch * g.c_bstride + row;
    if (kOut == kF32 && g.L > 0) {
      const int n = row & mask;
      if (n == mask) continue;  // the spare column of each tree
      out_row = batch * g.c_bstride + static_cast<int64_t>(row >> g.L) * g.Nn + n;
    }
#pragma unroll
    for (int j = 0; j < C::kTn; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * C::WN + j * 32 + q * 8 + (lane >> 5) * 4;
        if (col >= g.N) continue;
        if constexpr (kOut == kF32) {
          float* dst = static_cast<float*>(g.C) + ks * g.split_stride + out_row * g.ldc + col;
          *reinterpret_cast<float4*>(dst) = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                        acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        } else {
          uint16_t* dst = static_cast<uint16_t*>(g.C) + out_row * g.ldc + col;
          *reinterpret_cast<uint2*>(dst) =
              make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                         pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
        }
      }
    }
  }
}

// out[i] = sum over s < ks of part[s * n + i], in split order (n % 4 == 0).
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part,
                                                         float* __restrict__ out, int64_t n,
                                                         int ks) {
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x * 4) {
    float4 a = *reinterpret_cast<const float4*>(part + i);
    for (int s = 1; s < ks; ++s) {
      const float4 b = *reinterpret_cast<const float4*>(part + s * n + i);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    *reinterpret_cast<float4*>(out + i) = a;
  }
}

// dst[c][r] = src row r's element c (zero for rows without a source), for
// r < Rp, c < Cn; 64 x 64 tiles through LDS.  Source row of r: r itself if
// r < R (L = 0), else for the node layout (L > 0) p * Nn + n with
// p = r >> L, n = r & (2^L - 1) when n < 2^L - 1 and p < P.
__global__ __launch_bounds__(256) void transpose_rows_kernel(
    const uint16_t* __restrict__ src, int64_t ld_src, uint16_t* __restrict__ dst, int64_t ld_dst,
    int64_t R, int Cn, int L, int64_t Nn, int P) {
  __shared__ uint16_t tile[64][72];
  const int c0 = blockIdx.x * 64;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int tr = threadIdx.x >> 2;        // tile row (source row r0 + tr)
  const int tc = (threadIdx.x & 3) * 16;  // 16 columns
  const int64_t r = r0 + tr;
  int64_t srow = -1;
  if (L == 0) {
    srow = r < R ? r : -1;
  } else {
    const int64_t p = r >> L;
    const int64_t n = r & ((int64_t(1) << L) - 1);
    srow = (p < P && n < (int64_t(1) << L) - 1) ? p * Nn + n : -1;
  }
  uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
  if (srow >= 0 && c0 + tc < Cn) {
    v0 = ldg16(src + srow * ld_src + c0 + tc);
    v1 = ldg16(src + srow * ld_src + c0 + tc + 8);
  }
  *reinterpret_cast<uint4*>(&tile[tr][tc]) = v0;
  *reinterpret_cast<uint4*>(&tile[tr][tc + 8]) = v1;
  __syncthreads();
  const int oc = threadIdx.x >> 2;        // output row c0 + oc
  const int orr = (threadIdx.x & 3) * 16;  // 16 consecutive r
  if (c0 + oc >= Cn) return;
  uint16_t w[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) w[e] = tile[orr + e][oc];
  uint16_t* o = dst + static_cast<int64_t>(c0 + oc) * ld_dst + r0 + orr;
  *reinterpret_cast<uint4*>(o) = make_uint4(w[0] | (uint32_t(w[1]) << 16), w[2] | (uint32_t(w[3]) << 16),
                                            w[4] | (uint32_t(w[5]) << 16), w[6] | (uint32_t(w[7]) << 16));
  *reinterpret_cast<uint4*>(o + 8) = make_uint4(w[8] | (uint32_t(w[9]) << 16), w[10] | (uint32_t(w[11]) << 16),
                                                w[12] | (uint32_t(w[13]) << 16), w[14] | (uint32_t(w[15]) << 16));
}

// One thread per (tree p, token t < Tp): from the routing records, dH^T
// (fp32 [K][Tp], so that the lanes of a wave read consecutive tokens of one
// column) and the tree's v rows (staged in LDS), the path's da and GELU
// terms; writes
// the masked rows DA[t][p*2^L ..], the transposed columns DA^T, G^T, H^T
// and dS^T at token t (zeros for padding tokens t >= T), and db through an
// LDS reduction per node.
__global__ __launch_bounds__(256) void bwd_paths_kernel(
    const float* __restrict__ rec_logit, const int32_t* __restrict__ rec_next,
    const uint16_t* __restrict__ V, const float* __restrict__ dHt, uint16_t* __restrict__ DA,
    uint16_t* __restrict__ DAt, uint16_t* __restrict__ Gt, uint16_t* __restrict__ Ht,
    uint16_t* __restrict__ dSt, float* __restrict__ db, int T, int Tp, int P, int D, int h,
    int64_t N, int post) {
  extern __shared__ __align__(16) unsigned char bp_lds[];
  const int L = D + 1;
  const int cpt = 1 << L;
  uint16_t* Vs = reinterpret_cast<uint16_t*>(bp_lds);
  float* dbs = reinterpret_cast<float*>(bp_lds + ((size_t(N) * h * 2 + 15) / 16) * 16);
  const int p = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const uint16_t* Vp = V + static_cast<int64_t>(p) * N * h;
  // The tree's V rows are contiguous: copied straight into LDS, 1 KB per
  // wave-wide load (lane i at byte 16 i), all in flight together.
  {
    const unsigned char* src = reinterpret_cast<const unsigned char*>(Vp);
    const int total = static_cast<int>(N) * h * 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    for (int base = wave * 1024; base < total; base += 4 * 1024)
      if (base + lane * 16 < total)
        __builtin_amdgcn_global_load_lds(src + base + lane * 16,
                                         reinterpret_cast<unsigned char*>(Vs) + base, 16, 0, 0);
  }
  for (int c = threadIdx.x; c < cpt; c += 256) dbs[c] = 0.0f;
  wait_vmcnt<0>();
  __syncthreads();

  const bool live = t < T;
  int node[8];
  float a[8], g[8];
  const int leaf = live ? rec_next[static_cast<int64_t>(p) * T + t] : 0;
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    node[l] = live && l < L ? ((leaf + 1) >> (D - l)) - 1 : 0;
    a[l] = (live && l < L) ? rec_logit[(static_cast<int64_t>(p) * T + t) * L + l] : 0.0f;
    g[l] = 0.0f;
  }
  // Weight of each level's v row: GELU(a), or a itself for FFFpost; formed
  // once per level and reused by every column below.
  float gw[8];
#pragma unroll
  for (int l = 0; l < 8; ++l) gw[l] = post ? a[l] : gelu_tanh(a[l]);
  const float* dHp = dHt + static_cast<int64_t>(p) * h * Tp + (live ? t : 0);
  for (int j0 = 0; j0 < h; j0 += 8) {
    float dj[8], hj[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dj[e] = dHp[static_cast<int64_t>(j0 + e) * Tp];
    if (!live) {
#pragma unroll
      for (int e = 0; e < 8; ++e) dj[e] = 0.0f;
    }
    float sj[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sj[e] = 0.0f;
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      if (l >= L) break;
      const uint4 u = *reinterpret_cast<const uint4*>(Vs + static_cast<size_t>(node[l]) * h + j0);
      const float v[8] = {bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y),
                          bf16lo(u.z), bf16hi(u.z), bf16lo(u.w), bf16hi(u.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) sj[e] += gw[l] * v[e];
    }
    // FFF: sj is H; FFF-post: sj is s, H = GELU(s), dS = GELU'(s) dH.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hj[e] = post ? gelu_tanh(sj[e]) : sj[e];
      if (post) dj[e] *= gelu_tanh_grad(sj[e]);
    }
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      if (l >= L) break;
      const uint4 u = *reinterpret_cast<const uint4*>(Vs + static_cast<size_t>(node[l]) * h + j0);
      g[l] += dj[0] * bf16lo(u.x) + dj[1] * bf16hi(u.x) + dj[2] * bf16lo(u.y) +
              dj[3] * bf16hi(u.y) + dj[4] * bf16lo(u.z) + dj[5] * bf16hi(u.z) +
              dj[6] * bf16lo(u.w) + dj[7] * bf16hi(u.w);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t row = static_cast<int64_t>(p) * h + j0 + e;
      Ht[row * Tp + t] = live ? f32_to_bf16(hj[e]) : 0;
      dSt[row * Tp + t] = live ? f32_to_bf16(dj[e]) : 0;
    }
  }
  float da[8];
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    da[l] = (live && l < L) ? (post ? g[l] : g[l] * gelu_tanh_grad(a[l])) : 0.0f;
    if (live && l < L) atomicAdd(dbs + node[l], da[l]);
  }
  // Masked rows and columns: node c (heap order) holds the value of the
  // level it sits on if the path passes through it.
  for (int c0 = 0; c0 < cpt; c0 += 8) {
    uint16_t dv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      const int lvl = 31 - __clz(c + 1);
      float vd = 0.0f, vg = 0.0f;
#pragma unroll
      for (int l = 0; l < 8; ++l)
        if (l == lvl && l < L && node[l] == c) {
          vd = da[l];
          vg = gw[l];
        }
      if (!live) vd = vg = 0.0f;
      dv[e] = f32_to_bf16(vd);
      const int64_t col = static_cast<int64_t>(p) * cpt + c;
      DAt[col * Tp + t] = dv[e];
      Gt[col * Tp + t] = f32_to_bf16(vg);
    }
    if (live)
      *reinterpret_cast<uint4*>(DA + static_cast<int64_t>(t) * P * cpt + static_cast<int64_t>(p) * cpt + c0) =
          make_uint4(dv[0] | (uint32_t(dv[1]) << 16), dv[2] | (uint32_t(dv[3]) << 16),
                     dv[4] | (uint32_t(dv[5]) << 16), dv[6] | (uint32_t(dv[7]) << 16));
  }
  __syncthreads();
  for (int c = threadIdx.x; c < cpt - 1; c += 256)
    if (dbs[c] != 0.0f) atomicAdd(db + static_cast<int64_t>(p) * N + c, dbs[c]);
}

}  // namespace

hipError_t launch_fill_f32(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_f32_kernel<<<grid_for(n), 256, 0, st>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_backward_generic(const Dims& s, const void* x, const void* W, const void* V,
                                   const void* Wout, const void* dy, void* dx, float* dW, float* db,
                                   float* dV, float* dWout, const float* logits,
                                   const int32_t* leaf, float* dH, float* Hf, float* dxacc,
                                   hipStream_t st) {
  if (s.dtype == 0)
    return backward_generic_t<float>(s, x, W, V, Wout, dy, dx, dW, db, dV, dWout, logits, leaf, dH,
                                     Hf, dxacc, st);
  return backward_generic_t<uint16_t>(s, x, W, V, Wout, dy, dx, dW, db, dV, dWout, logits, leaf,
                                      dH, Hf, dxacc, st);
}

namespace {

template <class C, int kOut>
hipError_t launch_gemm_nt(GemmArgs g, int batches, hipStream_t st) {
  {
    const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(gemm_nt_kernel<C, kOut>),
                                          static_cast<int>(C::kLdsBytes));
    if (e != hipSuccess) return e;
  }
  g.tiles_m = (g.M + C::BM - 1) / C::BM;
  g.tiles_n = (g.N + C::BN - 1) / C::BN;
  const int blocks = g.tiles_m * g.tiles_n * g.ksplit * batches;
  gemm_nt_kernel<C, kOut><<<dim3(blocks), dim3(C::kThreads), C::kLdsBytes, st>>>(g);
  return hipGetLastError();
}

// Splits of the token dimension so that a float32 product covers the 256
// compute units (each split a multiple of the 32-wide k step).
int token_splits(int tiles, int64_t Tp) {
  int ks = 1;
  while (tiles * ks < 256 && ks < 8 && (Tp / 32) % (2 * ks) == 0) ks *= 2;
  return ks;
}

hipError_t transpose_rows(const uint16_t* src, int64_t ld_src, uint16_t* dst, int64_t ld_dst,
                          int64_t R, int64_t Rp, int Cn, int L, int64_t Nn, int P,
                          hipStream_t st) {
  transpose_rows_kernel<<<dim3((Cn + 63) / 64, static_cast<unsigned>(Rp / 64)), 256, 0, st>>>(
      src, ld_src, dst, ld_dst, R, Cn, L, Nn, P);
  return hipGetLastError();
}

// Splits of the token dimension of the dW, dW_out and dV products.
struct BwdSplits {
  int w, o, v;
};
BwdSplits bwd_splits(const Dims& s) {
  const int L = s.D + 1;
  const int64_t Tp = (s.T + 255) / 256 * 256;
  const int cols = s.P << L;
  BwdSplits k;
  k.w = token_splits(((cols + 255) / 256) * ((s.d + 255) / 256), Tp);
  k.o = token_splits(static_cast<int>(((s.K + 255) / 256) * ((s.d + 255) / 256)), Tp);
  k.v = token_splits(s.P * (((1 << L) + 127) / 128) * ((s.h + 127) / 128), Tp);
  return k;
}

hipError_t sum_splits(const float* part, float* out, int64_t n, int ks, hipStream_t st) {
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  sum_splits_kernel<<<dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks)), 256, 0, st>>>(part, out,
                                                                                            n, ks);
  return hipGetLastError();
}

size_t paths_lds(const Dims& s) {
  return (size_t(s.N) * s.h * 2 + 15) / 16 * 16 + (size_t(1) << (s.D + 1)) * 4;
}

}  // namespace

bool backward_mfma_supported(const Dims& s) {
  const int L = s.D + 1;
  return s.dtype == 1 && L >= 3 && L <= 8 && route_top_supported(s, L) && s.d % 64 == 0 &&
         s.h % 64 == 0 && (int64_t(s.P) << L) % 64 == 0 && paths_lds(s) <= 64 * 1024 &&
         s.T >= 1;
}

BwdMfmaLayout backward_mfma_layout(const Dims& s) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const int L = s.D + 1;
  const size_t cols = size_t(s.P) << L;
  const size_t Tp = (size_t(s.T) + 255) / 256 * 256;
  BwdMfmaLayout B;
  size_t off = 0;
  B.Tp = static_cast<int64_t>(Tp);
  B.logits = off; off = up(off + size_t(s.T) * s.P * L * 4);
  B.next = off;   off = up(off + size_t(s.T) * s.P * 4);
  B.xT = off;     off = up(off + size_t(s.d) * Tp * 2);
  B.dyT = off;    off = up(off + size_t(s.d) * Tp * 2);
  B.dH = off;     off = up(off + size_t(s.K) * Tp * 4);  // dH^T
  B.DA = off;     off = up(off + size_t(s.T) * cols * 2);
  B.DAt = off;    off = up(off + cols * Tp * 2);
  B.Gt = off;     off = up(off + cols * Tp * 2);
  B.Ht = off;     off = up(off + size_t(s.K) * Tp * 2);
  B.dSt = off;    off = up(off + size_t(s.K) * Tp * 2);
  B.WTn = off;    off = up(off + size_t(s.d) * cols * 2);
  // Partial products of the split token dimension (the largest of the three).
  const BwdSplits k = bwd_splits(s);
  size_t part = 0;
  const size_t nW = size_t(s.P) * s.N * s.d, nO = size_t(s.K) * s.d, nV = size_t(s.P) * s.N * s.h;
  if (k.w > 1) part = std::max(part, k.w * nW);
  if (k.o > 1) part = std::max(part, k.o * nO);
  if (k.v > 1) part = std::max(part, k.v * nV);
  B.part = off;   off = up(off + part * 4);
  B.total = off;
  return B;
}

hipError_t launch_backward_mfma(const Dims& s, const void* x, const void* W, const void* b,
                                const void* V, const void* Wout, const void* dy, void* dx,
                                float* dW, float* db, float* dV, float* dWout, void* ws,
                                hipStream_t st) {
  const int L = s.D + 1;
  const int cols = s.P << L;
  const BwdMfmaLayout B = backward_mfma_layout(s);
  const int64_t Tp = B.Tp;
  char* w = static_cast<char*>(ws);
  float* logits = reinterpret_cast<float*>(w + B.logits);
  int32_t* next = reinterpret_cast<int32_t*>(w + B.next);
  uint16_t* xT = reinterpret_cast<uint16_t*>(w + B.xT);
  uint16_t* dyT = reinterpret_cast<uint16_t*>(w + B.dyT);
  float* dH = reinterpret_cast<float*>(w + B.dH);
  uint16_t* DA = reinterpret_cast<uint16_t*>(w + B.DA);
  uint16_t* DAt = reinterpret_cast<uint16_t*>(w + B.DAt);
  uint16_t* Gt = reinterpret_cast<uint16_t*>(w + B.Gt);
  uint16_t* Ht = reinterpret_cast<uint16_t*>(w + B.Ht);
  uint16_t* dSt = reinterpret_cast<uint16_t*>(w + B.dSt);
  uint16_t* WTn = reinterpret_cast<uint16_t*>(w + B.WTn);
  const uint16_t* x16 = static_cast<const uint16_t*>(x);
  const uint16_t* dy16 = static_cast<const uint16_t*>(dy);
  hipError_t e;
#define FFF_TRY(...) \
  if ((e = (__VA_ARGS__)) != hipSuccess) return e
  float* part = reinterpret_cast<float*>(w + B.part);
  const BwdSplits k = bwd_splits(s);
  const int64_t nW = int64_t(s.P) * s.N * s.d, nO = s.K * s.d, nV = int64_t(s.P) * s.N * s.h;
  // db gathers atomically; dW, dW_out and dV are written in full below.
  FFF_TRY(launch_fill_f32(db, int64_t(s.P) * s.N, st));
  FFF_TRY(launch_route_top(s, L, L, x, W, b, logits, next, st));
  FFF_TRY(transpose_rows(x16, s.d, xT, Tp, s.T, Tp, s.d, 0, 0, 0, st));
  FFF_TRY(transpose_rows(dy16, s.d, dyT, Tp, s.T, Tp, s.d, 0, 0, 0, st));
  FFF_TRY(transpose_rows(static_cast<const uint16_t*>(W), s.d, WTn, cols, cols, cols, s.d, L, s.N,
                         s.P, st));
  GemmArgs g{};
  // dH^T = W_out . dy^T  [K, Tp] (columns t >= T are not written and not read)
  g.A = static_cast<const uint16_t*>(Wout); g.lda = s.d; g.B = dy16; g.ldb = s.d;
  g.C = dH; g.ldc = Tp; g.M = static_cast<int>(s.K); g.N = static_cast<int>(s.T); g.Kk = s.d;
  g.ksplit = 1;
  FFF_TRY(launch_gemm_nt<BwdTile, kF32>(g, 1, st));
  bwd_paths_kernel<<<dim3(static_cast<unsigned>(Tp / 256), static_cast<unsigned>(s.P)), 256,
                     paths_lds(s), st>>>(logits, next, static_cast<const uint16_t*>(V), dH, DA,
                                         DAt, Gt, Ht, dSt, db, static_cast<int>(s.T),
                                         static_cast<int>(Tp), s.P, s.D, s.h, s.N, s.variant);
  FFF_TRY(hipGetLastError());
  // dx = DA . W_top  [T, d]
  g = GemmArgs{};
  g.A = DA; g.lda = cols; g.B = WTn; g.ldb = cols; g.C = dx; g.ldc = s.d;
  g.M = static_cast<int>(s.T); g.N = s.d; g.Kk = cols; g.ksplit = 1;
  FFF_TRY(launch_gemm_nt<BwdTile, kBf16>(g, 1, st));
  // dW = DA^T . x  [P*2^L -> P*N, d]
  g = GemmArgs{};
  g.A = DAt; g.lda = Tp; g.B = xT; g.ldb = Tp; g.C = dW; g.ldc = s.d;
  g.M = cols; g.N = s.d; g.L = L; g.Nn = s.N;
  g.ksplit = k.w;
  g.Kk = static_cast<int>(Tp / g.ksplit);
  if (k.w > 1) g.C = part, g.split_stride = nW;
  FFF_TRY(launch_gemm_nt<BwdTile, kF32>(g, 1, st));
  if (k.w > 1) FFF_TRY(sum_splits(part, dW, nW, k.w, st));
  // dW_out = H^T . dy  [K, d]
  g = GemmArgs{};
  g.A = Ht; g.lda = Tp; g.B = dyT; g.ldb = Tp; g.C = dWout; g.ldc = s.d;
  g.M = static_cast<int>(s.K); g.N = s.d;
  g.ksplit = k.o;
  g.Kk = static_cast<int>(Tp / g.ksplit);
  if (k.o > 1) g.C = part, g.split_stride = nO;
  FFF_TRY(launch_gemm_nt<BwdTile, kF32>(g, 1, st));
  if (k.o > 1) FFF_TRY(sum_splits(part, dWout, nO, k.o, st));
  // dV_p = G_p^T . dS_p  [2^L -> N, h], one batch per tree
  g = GemmArgs{};
  g.A = Gt; g.lda = Tp; g.a_bstride = int64_t(1) << L;
  g.B = dSt; g.ldb = Tp; g.b_bstride = s.h;
  g.C = dV; g.ldc = s.h; g.c_bstride = s.N; g.M = 1 << L; g.N = s.h; g.L = L; g.Nn = s.N;
  g.ksplit = k.v;
  g.Kk = static_cast<int>(Tp / g.ksplit);
  if (k.v > 1) g.C = part, g.split_stride = nV;
  FFF_TRY(launch_gemm_nt<BwdSmallTile, kF32>(g, s.P, st));
  if (k.v > 1) FFF_TRY(sum_splits(part, dV, nV, k.v, st));
#undef FFF_TRY
  return hipSuccess;
}

}  // namespace fff
