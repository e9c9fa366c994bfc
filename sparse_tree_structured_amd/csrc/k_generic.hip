// Generic FFF forward kernels: correct for every shape and both dtypes.
//
// The layer follows "Dynamic sparsity in tree-structured feed-forward layers
// at scale" (gist.science explainer, section 2): each token walks one
// root-to-leaf path per tree, the sign of the node logit choosing the child,
// and the visited nodes' GELU(a) * v_n are summed (GELU before the sum,
// section 3.C); the tree outputs are concatenated and projected (Figure 1(c)
// caption on the paper's page).
//
// Three kernels: one wavefront per (token, tree) walks the tree and keeps the
// D+1 logits; one thread per element of H sums GELU(a) * v over the path; a
// tiled fp32 matrix product applies W_out.
#include "common.hpp"
#include "launch.hpp"

namespace fff {
namespace {

template <typename E>
__global__ __launch_bounds__(256) void route_generic_kernel(
    const E* __restrict__ x, const E* __restrict__ W, const E* __restrict__ b,
    float* __restrict__ logits, int32_t* __restrict__ path_out, int32_t* __restrict__ leaf_ws,
    int64_t T, int d, int P, int D, int64_t N, const uint8_t* __restrict__ alive) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (pair >= T * P) return;  // whole wavefront leaves together
  const int64_t t = pair / P;
  const int p = static_cast<int>(pair % P);
  const E* xt = x + t * d;
  const E* Wp = W + static_cast<int64_t>(p) * N * d;
  int64_t n = 0;
  for (int level = 0; level <= D; ++level) {
    const E* w = Wp + n * d;
    float acc = 0.0f;
    for (int i = lane; i < d; i += kWave) acc += Elem<E>::ld(xt, i) * Elem<E>::ld(w, i);
    const float a = wave_sum(acc) + Elem<E>::ld(b, static_cast<size_t>(p) * N + n);
    if (lane == 0) logits[pair * (D + 1) + level] = a;
    if (level < D) {
      int r = go_right(a);
      // Static pruning: a step into a pruned child goes to the sibling.
      if (alive && !alive[static_cast<int64_t>(p) * N + 2 * n + 1 + r]) r ^= 1;
      n = 2 * n + 1 + r;
    }
  }
  if (lane == 0) {
    const int32_t leaf = static_cast<int32_t>(n - ((int64_t(1) << D) - 1));
    leaf_ws[pair] = leaf;
    if (path_out) path_out[pair] = leaf;
  }
}

template <typename E>
__global__ __launch_bounds__(256) void hbuild_generic_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ leaf_ws, const E* __restrict__ V,
    E* __restrict__ H, int64_t T, int P, int D, int h, int64_t N, int post) {
  const int64_t K = static_cast<int64_t>(P) * h;
  const int64_t total = T * K;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
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
    Elem<E>::st(H, e, post ? gelu_tanh(acc) : acc);
  }
}

// C[M,Nc] = A[M,K] . B[K,Nc]; 64x64 tile per 256 threads, 4x4 outputs each.
template <typename E>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const E* __restrict__ A,
                                                           const E* __restrict__ B,
                                                           E* __restrict__ C, int64_t M,
                                                           int64_t K, int64_t Nc) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int tx = threadIdx.x & 15;  // column group
  const int ty = threadIdx.x >> 4;  // row group
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t col0 = static_cast<int64_t>(blockIdx.y) * 64;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int kk = e / 64, mm = e % 64;
      const int64_t r = row0 + mm, k = k0 + kk;
      As[kk][mm] = (r < M && k < K) ? Elem<E>::ld(A, r * K + k) : 0.0f;
      const int64_t c = col0 + mm;
      Bs[kk][mm] = (c < Nc && k < K) ? Elem<E>::ld(B, k * Nc + c) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * bb[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t r = row0 + ty * 4 + i, c = col0 + tx * 4 + j;
      if (r < M && c < Nc) Elem<E>::st(C, r * Nc + c, acc[i][j]);
    }
}

}  // namespace

hipError_t launch_route_generic(const Dims& s, const void* x, const void* W, const void* b,
                                float* logits, int32_t* path_out, int32_t* leaf_ws,
                                hipStream_t st) {
  const int64_t pairs = s.T * s.P;
  const dim3 grid(static_cast<unsigned>((pairs + 3) / 4));
  if (s.dtype == 0)
    route_generic_kernel<float><<<grid, 256, 0, st>>>(
        static_cast<const float*>(x), static_cast<const float*>(W), static_cast<const float*>(b),
        logits, path_out, leaf_ws, s.T, s.d, s.P, s.D, s.N, s.prune ? s.prune->alive : nullptr);
  else
    route_generic_kernel<uint16_t><<<grid, 256, 0, st>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W),
        static_cast<const uint16_t*>(b), logits, path_out, leaf_ws, s.T, s.d, s.P, s.D, s.N,
        s.prune ? s.prune->alive : nullptr);
  return hipGetLastError();
}

hipError_t launch_hbuild_generic(const Dims& s, const float* logits, const int32_t* leaf_ws,
                                 const void* V, void* H, hipStream_t st) {
  const int64_t total = s.T * s.K;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (s.dtype == 0)
    hbuild_generic_kernel<float><<<static_cast<unsigned>(blocks), 256, 0, st>>>(
        logits, leaf_ws, static_cast<const float*>(V), static_cast<float*>(H), s.T, s.P, s.D,
        s.h, s.N, s.variant);
  else
    hbuild_generic_kernel<uint16_t><<<static_cast<unsigned>(blocks), 256, 0, st>>>(
        logits, leaf_ws, static_cast<const uint16_t*>(V), static_cast<uint16_t*>(H), s.T, s.P,
        s.D, s.h, s.N, s.variant);
  return hipGetLastError();
}

hipError_t launch_project_generic(const Dims& s, const void* H, const void* Wout, void* y,
                                  hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((s.T + 63) / 64), static_cast<unsigned>((s.d + 63) / 64));
  if (s.dtype == 0)
    gemm_generic_kernel<float><<<grid, 256, 0, st>>>(static_cast<const float*>(H),
                                                     static_cast<const float*>(Wout),
                                                     static_cast<float*>(y), s.T, s.K, s.d);
  else
    gemm_generic_kernel<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(H),
                                                        static_cast<const uint16_t*>(Wout),
                                                        static_cast<uint16_t*>(y), s.T, s.K, s.d);
  return hipGetLastError();
}

}  // namespace fff
