// Device helpers shared by the gfx950 kernels of the FFF forward pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fff {

constexpr int kWave = 64;  // CDNA wavefront width

// bfloat16 is carried as its raw 16 bits.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 conversions use gfx950's v_cvt_pk_bf16_f32 (round to
// nearest even, NaN stays NaN), which the compiler emits for these casts.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two bf16 in one dword: low half is the lower index.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// GELU, tanh form: 0.5 a (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))).
__device__ __forceinline__ float gelu_tanh(float a) {
  const float k0 = 0.7978845608028654f;
  const float k1 = 0.044715f;
  return 0.5f * a * (1.0f + tanhf(k0 * (a + k1 * a * a * a)));
}

// Storage element <-> fp32.
template <typename E> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Routing decision: a < 0 goes left (0); 0, -0 and NaN go right (1).
__device__ __forceinline__ int go_right(float a) { return !(a < 0.0f); }

}  // namespace fff
