// Matrix-core tile machinery shared by the dense kernels (gfx950, bf16 in,
// fp32 accumulate).
//
// A workgroup computes C[BM x BN] = A[BM x K] . B[K x BN]; its wavefronts are
// arranged kWavesM x kWavesN, each owning WM x WN = kTm x kTn blocks of
// v_mfma_f32_32x32x16_bf16.  K advances by BK through two LDS buffers: global
// loads of the next step are issued before the matrix-core work of the
// current one, then written to the other buffer.
//
// Both operands sit in LDS K-contiguous, one row per output row / column,
// rows padded by 16 bytes so that the 16-byte operand reads of 8 consecutive
// lanes cover all banks.  The MFMA is issued with the B fragment first, so an
// accumulator block is the transposed C block: lane l holds C row
// (block row + l % 32) and columns 8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
#pragma once

#include "common.hpp"

namespace fff {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int kWavesM = BM / WM;
  static constexpr int kWavesN = BN / WN;
  static constexpr int kThreads = kWavesM * kWavesN * kWave;
  static constexpr int kLd = BK + 8;  // LDS row pitch in elements
  static constexpr int kTm = WM / 32;
  static constexpr int kTn = WN / 32;
  static constexpr int kStage = (BM + BN) * kLd;  // elements per LDS buffer
  static constexpr size_t kLdsBytes = 2 * kStage * sizeof(uint16_t);
  static_assert(BK % 16 == 0 && WM % 32 == 0 && WN % 32 == 0, "MFMA block shape");
};

// Rows of a K-contiguous matrix, gathered through a row-address callback:
// row_ptr(i) for i in [0, ROWS) returns the start of that row (already
// clamped to valid memory by the caller).
template <int ROWS, int BK, int THREADS>
struct RowLoader {
  static constexpr int kChunks = ROWS * BK / 8 / THREADS;  // 16-byte pieces per thread
  static_assert(ROWS * BK / 8 % THREADS == 0, "rows must split evenly");
  uint4 r[kChunks];

  template <class RowPtr>
  __device__ __forceinline__ void load(const RowPtr& row_ptr, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * THREADS;
      const int row = c / (BK / 8);
      const int kc = c % (BK / 8);
      r[i] = ldg16(row_ptr(row) + k0 + kc * 8);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int ld, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * THREADS;
      const int row = c / (BK / 8);
      const int kc = c % (BK / 8);
      *reinterpret_cast<uint4*>(lds + row * ld + kc * 8) = r[i];
    }
  }
};

// Accumulator helpers.
template <class C>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[C::kTm][C::kTn]) {
#pragma unroll
  for (int i = 0; i < C::kTm; ++i)
#pragma unroll
    for (int j = 0; j < C::kTn; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// Matrix-core work on one LDS buffer (As: BM rows, Bs: BN rows, both [row][k]).
template <class C>
__device__ __forceinline__ void mma_stage(f32x16_t (&acc)[C::kTm][C::kTn], const uint16_t* As,
                                          const uint16_t* Bs, int wm, int wn, int lane) {
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < C::BK; kk += 16) {
    bf16x8_t af[C::kTm], bfr[C::kTn];
#pragma unroll
    for (int i = 0; i < C::kTm; ++i)
      af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * C::WM + i * 32 + lrow) * C::kLd + kk + lk);
#pragma unroll
    for (int j = 0; j < C::kTn; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * C::WN + j * 32 + lrow) * C::kLd + kk + lk);
#pragma unroll
    for (int i = 0; i < C::kTm; ++i)
#pragma unroll
      for (int j = 0; j < C::kTn; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  }
}

// Full K loop.  ALoad / BLoad provide load(k0) (global -> registers) and
// store(lds, ld) (registers -> LDS) for their operand.
template <class C, class ALoad, class BLoad>
__device__ __forceinline__ void gemm_mainloop(f32x16_t (&acc)[C::kTm][C::kTn], uint16_t* smem,
                                              int K, ALoad& la, BLoad& lb) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / C::kWavesN;
  const int wn = wave % C::kWavesN;
  zero_acc<C>(acc);
  const int ksteps = K / C::BK;
  la.load(0);
  lb.load(0);
  la.store(smem, C::kLd);
  lb.store(smem + C::BM * C::kLd, C::kLd);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < ksteps) {
      la.load((ks + 1) * C::BK);
      lb.load((ks + 1) * C::BK);
    }
    const uint16_t* As = smem + cur * C::kStage;
    mma_stage<C>(acc, As, As + C::BM * C::kLd, wm, wn, lane);
    if (ks + 1 < ksteps) {
      uint16_t* Asn = smem + (cur ^ 1) * C::kStage;
      la.store(Asn, C::kLd);
      lb.store(Asn + C::BM * C::kLd, C::kLd);
    }
    __syncthreads();
  }
}

// XCD-aware tile order: hardware sends workgroup b to XCD b % 8.  Each XCD
// gets a contiguous range of logical tiles (row-panel major), so operand
// panels are fetched from HBM about once per XCD and the tiles an XCD runs
// together share k-slices in its L2.
__device__ __forceinline__ int xcd_logical_tile(int b, int nblk) {
  return (nblk % 8) != 0 ? b : (b % 8) * (nblk / 8) + (b / 8);
}

}  // namespace fff
