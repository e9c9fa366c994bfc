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

// ---------------------------------------------------------------------------
// Direct-to-LDS main loop (A rows K-contiguous; B as K-contiguous rows of
// the output columns, or k-major: KMajorBOp below).
//
// Each K step of 32 lives in one of kStages LDS buffers; the buffers are
// filled with global_load_lds_dwordx4 (16 bytes per lane straight into LDS,
// no register staging), kStages-1 steps ahead of the matrix-core work.  One
// wave-wide load fills 1 KB = 16 rows x 64 bytes.  A row's four 16-byte
// chunks are stored XOR-swizzled, chunk c of row r at slot c ^ f(r) with
// f(r) = (r >> 2) & 3.  The operand reads (32 consecutive rows, one chunk per
// half wavefront) are then free of LDS bank conflicts; this choice was
// measured with the SQ_LDS_BANK_CONFLICT counter on gfx950, where other
// XOR patterns that look conflict-free on paper give 2-way conflicts.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_, int STAGES_>
struct DirectCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 32, WM = WM_, WN = WN_;
  static constexpr int kStages = STAGES_;
  static constexpr int kWavesM = BM / WM;
  static constexpr int kWavesN = BN / WN;
  static constexpr int kWaves = kWavesM * kWavesN;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kTm = WM / 32;
  static constexpr int kTn = WN / 32;
  static constexpr int kRowBytes = BK * 2;  // 64
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr size_t kLdsBytes = size_t(kStages) * kStageBytes;
  static constexpr int kALoads = BM / 16 / kWaves;  // wave-wide loads per stage
  static constexpr int kBLoads = BN / 16 / kWaves;
  static_assert(BM % (16 * kWaves) == 0 && BN % (16 * kWaves) == 0, "rows split over waves");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "MFMA block shape");
};

__device__ __forceinline__ int lds_swz(int r) { return (r >> 2) & 3; }

// Wait until at most n vector-memory operations of this wave are in flight
// (lgkm and exp counters left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most min(later, MAXLATER) stages of PER loads each are in
// flight (the immediate of s_waitcnt must be a compile-time constant).
template <int PER, int MAXLATER>
__device__ __forceinline__ void wait_stages(int later) {
  if constexpr (MAXLATER <= 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= MAXLATER)
      wait_vmcnt<MAXLATER * PER>();
    else
      wait_stages<PER, MAXLATER - 1>(later);
  }
}

// Issue the loads of one K step (k0) into stage buffer `buf` for ROWS rows
// starting at LDS byte offset `base`.  row_ptr(i) gives row i's start.
template <class C, int ROWS, class RowPtr>
__device__ __forceinline__ void direct_load_rows(unsigned char* lds, int base, const RowPtr& row_ptr,
                                                 int k0, int wave, int lane) {
  constexpr int kLoads = ROWS / 16 / C::kWaves;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int r0 = (wave * kLoads + j) * 16;
    const int r = r0 + (lane >> 2);
    const int chunk = (lane & 3) ^ lds_swz(r);
    const uint16_t* g = row_ptr(r) + k0 + chunk * 8;
    __builtin_amdgcn_global_load_lds(g, lds + base + r0 * C::kRowBytes, 16, 0, 0);
  }
}

// The same copy (16 bytes per lane into lds_dst + 16 * lane, lds_dst
// wave-uniform) written as inline assembly.  The compiler then does not know
// that the instruction writes LDS, so it does not hold later LDS reads
// behind it (it does so, with a full vmcnt(0), before every
// ds_read_b64_tr_b16 that follows a global_load_lds it issued itself); the
// caller waits for the copies with explicit s_waitcnt vmcnt, as the
// pipelined loops below do anyway.  M0 holds the LDS base during the copy
// and is restored afterwards; one wait state separates the M0 write from
// the copy.  The asm has no outputs but the saved M0, so no register is
// left pending.
__device__ __forceinline__ void dma16_asm(const void* g, const unsigned char* lds_dst) {
  // The low 32 bits of a generic LDS address are its LDS offset.
  const uint32_t m =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_dst)));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(m)
      : "memory");
}

template <class C, int ROWS, class RowPtr>
__device__ __forceinline__ void direct_load_rows_asm(unsigned char* lds, int base,
                                                     const RowPtr& row_ptr, int k0, int wave,
                                                     int lane, int64_t kmul) {
  constexpr int kLoads = ROWS / 16 / C::kWaves;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int r0 = (wave * kLoads + j) * 16;
    const int r = r0 + (lane >> 2);
    const int chunk = (lane & 3) ^ lds_swz(r);
    dma16_asm(row_ptr(r) + k0 * kmul + chunk * 8, lds + base + r0 * C::kRowBytes);
  }
}

// The same loads with the 16-byte chunks swizzled by row bits SHIFT and
// SHIFT+1: chunk c of row r at slot c ^ ((r >> SHIFT) & 3).  For the
// 16 x 16 x 32 operand fetch (16 rows, one chunk per 16 lanes) SHIFT = 1 is
// the bank-conflict-free choice on gfx950 for any 16 rows whose low four
// bits differ (measured with SQ_LDS_BANK_CONFLICT; SHIFT = 2 gives 2-way
// conflicts there).
template <int SHIFT>
__device__ __forceinline__ int lds_swz_s(int r) { return (r >> SHIFT) & 3; }

template <class C, int ROWS, int SHIFT, class RowPtr>
__device__ __forceinline__ void direct_load_rows_s(unsigned char* lds, int base, const RowPtr& row_ptr,
                                                   int k0, int wave, int lane) {
  constexpr int kLoads = ROWS / 16 / C::kWaves;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int r0 = (wave * kLoads + j) * 16;
    const int r = r0 + (lane >> 2);
    const int chunk = (lane & 3) ^ lds_swz_s<SHIFT>(r);
    const uint16_t* g = row_ptr(r) + k0 + chunk * 8;
    __builtin_amdgcn_global_load_lds(g, lds + base + r0 * C::kRowBytes, 16, 0, 0);
  }
}

// Operand fragments of one 16-wide k sub-step (kk = 0 or 1) of a stage.
template <class C>
struct Frags {
  bf16x8_t a[C::kTm], b[C::kTn];
};

// B operand held as rows of the output columns (B^T, K-contiguous): row j of
// the stage's B block is output column j, 64 bytes of k.  row_ptr(j) gives
// column j's K-contiguous start (already clamped to valid memory).
template <class C, class RowPtr>
struct RowsB {
  static constexpr bool kAsmDma = false;  // A and B copies through the builtin
  const RowPtr& row_ptr;
  __device__ __forceinline__ void issue(unsigned char* lds, int base, int k0, int wave,
                                        int lane) const {
    direct_load_rows<C, C::BN>(lds, base, row_ptr, k0, wave, lane);
  }
  __device__ __forceinline__ bf16x8_t frag(const unsigned char* Bs, int kk, int wn, int j,
                                           int lane) const {
    const int r = wn * C::WN + j * 32 + (lane & 31);
    const int chunk = kk * 2 + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(Bs + r * C::kRowBytes + ((chunk ^ lds_swz(r)) << 4));
  }
};

// B operand in its natural k-major layout (row k holds consecutive output
// columns, row stride ld elements), as y = H . W_out has it.  The stage's B
// block is BK = 32 rows of BN columns (BN * 2 bytes each, whole 128-byte
// lines per load); 16-byte chunk c of row r sits at slot c ^ 4 (r & 3).
// A fragment wants eight k-consecutive values of one column per lane, which
// ds_read_b64_tr_b16 assembles from a k-major tile: within each 16-lane
// group, lane 4 jj + a addresses row kb + jj at columns cb + 4 a .. cb + 4 a + 3,
// and lane i receives element i % 4 of the words of lanes i / 4, 4 + i / 4,
// 8 + i / 4 and 12 + i / 4, i.e. column cb + i at rows kb .. kb + 3.  Two
// such reads (rows kb and kb + 4) make the eight values.  With the swizzle,
// the 32 lanes of a half wavefront read 64 distinct banks.
struct KMajorB {
  const uint16_t* p;  // element (k = 0, column n0) of the tile
  int ld;             // row stride in elements
  int ncols;          // valid columns from n0 (chunks past it read column n0)
};

template <class C>
struct KMajorBOp {
  static constexpr bool kAsmDma = true;  // A and B copies through dma16_asm
  static constexpr int kRow = C::BN * 2;       // LDS bytes per k row
  static constexpr int kLoads = C::BN / 16 / C::kWaves;  // 1 KB loads per wave per stage
  static_assert(C::BN >= 128 && (C::BN * 2) % 256 == 0, "swizzle spans 16 chunks per row");
  static_assert(C::BK * C::BN * 2 == C::BN * C::kRowBytes, "stage B block size");
  KMajorB b;
  __device__ __forceinline__ static int swz(int r) { return (r & 3) << 2; }
  __device__ __forceinline__ void issue(unsigned char* lds, int base, int k0, int wave,
                                        int lane) const {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int q = wave * kLoads + j;  // 1 KB piece of the stage's B block
      const int byte = q * 1024 + lane * 16;
      const int r = byte / kRow;
      const int c = ((byte % kRow) >> 4) ^ swz(r);
      const int col = c * 8 < b.ncols ? c * 8 : 0;
      dma16_asm(b.p + static_cast<size_t>(k0 + r) * b.ld + col, lds + base + q * 1024);
    }
  }
  __device__ __forceinline__ bf16x8_t frag(const unsigned char* Bs, int kk, int wn, int j,
                                           int lane) const {
    typedef short v4i16_t __attribute__((ext_vector_type(4)));
    typedef short v8i16_t __attribute__((ext_vector_type(8)));
    const int cb = wn * C::WN + j * 32 + (lane & 16);  // group's first column
    const int kb = kk * 16 + ((lane >> 5) << 3);       // group's first row
    const int jj = (lane >> 2) & 3;
    const int col = cb + ((lane & 3) << 2);
    const int r = kb + jj;  // (r + 4) & 3 == r & 3: one swizzle for both reads
    const int off = r * kRow + (((col >> 3) ^ swz(r)) << 4) + ((col & 7) << 1);
    typedef __attribute__((address_space(3))) v4i16_t* lds_v4_t;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_t)(Bs + off));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_t)(Bs + off + 4 * kRow));
    const v8i16_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

template <class C, class BOp>
__device__ __forceinline__ void read_frags(Frags<C>& f, const unsigned char* stage, int kk, int wm,
                                           int wn, int lane, const BOp& bop) {
  const unsigned char* As = stage;
  const unsigned char* Bs = stage + C::BM * C::kRowBytes;
  const int lrow = lane & 31;
  const int chunk = kk * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::kTm; ++i) {
    const int r = wm * C::WM + i * 32 + lrow;
    f.a[i] = *reinterpret_cast<const bf16x8_t*>(As + r * C::kRowBytes + ((chunk ^ lds_swz(r)) << 4));
  }
#pragma unroll
  for (int j = 0; j < C::kTn; ++j) f.b[j] = bop.frag(Bs, kk, wn, j, lane);
}

template <class C>
__device__ __forceinline__ void mma_frags(f32x16_t (&acc)[C::kTm][C::kTn], const Frags<C>& f) {
#pragma unroll
  for (int i = 0; i < C::kTm; ++i)
#pragma unroll
    for (int j = 0; j < C::kTn; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// Workgroup barrier that does not drain the loads still in flight for later
// stages (__syncthreads() would).  The empty asm statements keep the
// compiler from moving memory operations across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Full K loop (K % 32 == 0).  a_row(i), i < BM, returns the start of A row
// i (already clamped to valid memory), whose K step k0 begins k0 * a_kmul
// elements further (1 for K-contiguous rows; with the asm copies only, the
// row count for K-blocked rows, where each 32-wide K slice of every row is
// contiguous); bop stages and reads the B operand (RowsB or KMajorBOp).
//
// Schedule of iteration ks (stage buffer ks % S):
//   read fragments (ks, kk=1)            -- LDS reads overlap the MFMAs below
//   MFMAs on fragments (ks, kk=0)
//   wait for stage ks+1's loads; barrier; issue the loads of stage ks+S-1
//   read fragments (ks+1, kk=0)
//   MFMAs on fragments (ks, kk=1)
// so every fragment is read one MFMA group (16 MFMAs) before its use and the
// loads of a stage are issued S-2 iterations before it is needed.
template <class C, class ARow, class BOp>
__device__ __forceinline__ void gemm_mainloop_direct_op(f32x16_t (&acc)[C::kTm][C::kTn],
                                                        unsigned char* lds, int K,
                                                        const ARow& a_row, const BOp& bop,
                                                        int64_t a_kmul = 1) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / C::kWavesN;
  const int wn = wave % C::kWavesN;
  constexpr int S = C::kStages;
  static_assert(S >= 3 && S <= 6, "wait counts below cover three to six stages");
  constexpr int kPerStage = C::kALoads + C::kBLoads;  // loads per wave per stage
  zero_acc<C>(acc);
  const int nk = K / C::BK;
  auto issue = [&](int ks) {
    const int base = (ks % S) * C::kStageBytes;
    if constexpr (BOp::kAsmDma)
      direct_load_rows_asm<C, C::BM>(lds, base, a_row, ks * C::BK, wave, lane, a_kmul);
    else
      direct_load_rows<C, C::BM>(lds, base, a_row, ks * C::BK, wave, lane);
    bop.issue(lds, base + C::BM * C::kRowBytes, ks * C::BK, wave, lane);
  };
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s);
  // Stage 0 ready: at most stages 1 .. S-2 still in flight.
  wait_stages<kPerStage, S - 2>(nk - 1);
  stage_barrier();
  Frags<C> f0, f1;
  read_frags<C>(f0, lds, 0, wm, wn, lane, bop);
  for (int ks = 0; ks < nk; ++ks) {
    const unsigned char* cur = lds + (ks % S) * C::kStageBytes;
    read_frags<C>(f1, cur, 1, wm, wn, lane, bop);
    asm volatile("" ::: "memory");  // keep these reads ahead of the MFMAs below
    mma_frags<C>(acc, f0);
    if (ks + 1 < nk) {
      // Stage ks+1 ready: at most stages ks+2 .. ks+S-2 still in flight.
      wait_stages<kPerStage, S - 3>(nk - 2 - ks);
      stage_barrier();  // also: every wave is done with stage ks-1's buffer
      if (ks + S - 1 < nk) issue(ks + S - 1);
    }
    // Unconditional (after the last stage it reads a stale buffer and the
    // values go unused), so the wait before the MFMAs below can leave these
    // eight reads in flight on every path.
    read_frags<C>(f0, lds + ((ks + 1) % S) * C::kStageBytes, 0, wm, wn, lane, bop);
    asm volatile("" ::: "memory");
    mma_frags<C>(acc, f1);
  }
  __syncthreads();
}

// Both operands K-contiguous: b_row(j), j < BN, returns output column j's
// row start (already clamped to valid memory).
template <class C, class ARow, class BRow>
__device__ __forceinline__ void gemm_mainloop_direct(f32x16_t (&acc)[C::kTm][C::kTn],
                                                     unsigned char* lds, int K, const ARow& a_row,
                                                     const BRow& b_row) {
  gemm_mainloop_direct_op<C>(acc, lds, K, a_row, RowsB<C, BRow>{b_row});
}

// XCD-aware tile order: hardware sends workgroup b to XCD b % 8.  Each XCD
// gets a contiguous range of logical tiles (row-panel major), so operand
// panels are fetched from HBM about once per XCD and the tiles an XCD runs
// together share k-slices in its L2.
__device__ __forceinline__ int xcd_logical_tile(int b, int nblk) {
  return (nblk % 8) != 0 ? b : (b % 8) * (nblk / 8) + (b / 8);
}

}  // namespace fff
