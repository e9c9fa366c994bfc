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
#include "fff.h"

#include "common.hpp"
#include "launch.hpp"

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

}  // namespace fff
