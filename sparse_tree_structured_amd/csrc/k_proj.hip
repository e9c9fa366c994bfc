// Output projection of the FFF layer on gfx950 matrix cores.
//
// The tree outputs are concatenated and passed through one final linear
// projection (paper page, Figure 1(c) caption): y[T,d] = H[T,K] . W_out[K,d]
// with K = P*h.  bf16 operands, fp32 accumulation (v_mfma_f32_32x32x16_bf16),
// bf16 result rounded to nearest even.
//
// Tiling (mfma_tile.hpp): a workgroup owns a BM x BN tile of y, each of its
// four wavefronts a WM x WN sub-tile made of 32x32 MFMA blocks (4x4 blocks =
// 128x128 with 256 accumulator registers per lane in the large
// configuration, so every 16 B read from LDS feeds four matrix-core
// operations).
//
// H rows are K-contiguous and go to LDS unchanged.  W_out rows are
// d-contiguous, but an MFMA operand lane needs 8 consecutive K values of one
// column, so each thread loads a 4(K) x 8(d) block, transposes it in
// registers with byte permutes and writes it to LDS as [n][k].  Consecutive
// lanes take consecutive K blocks so those 8-byte LDS writes hit distinct
// banks.
//
// Accumulator blocks are transposed y blocks, so a lane holds four
// consecutive output columns of one row, packed into one 8-byte store.
//
// Large products take the multi-stage direct-to-LDS kernel instead: both
// operands go from global memory straight into LDS (H rows as they are,
// W_out as k rows of the tile's columns), and the W_out fragments are read
// out of LDS with ds_read_b64_tr_b16, which transposes 16-bit elements
// across lanes, so W_out is used in its own layout with no preparation pass.
//
// XCD-aware tile order: each XCD owns a contiguous range of row panels, so H
// is fetched once in total and W_out once per XCD.
#include "common.hpp"
#include "launch.hpp"
#include "mfma_tile.hpp"

namespace fff {
namespace {

// Low (or high) 16-bit halves of two dwords into one dword: (b.half << 16) | a.half.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ uint32_t word(const uint4& q, int i) {
  return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// A operand: rows of H (K-contiguous), rows past M clamped to M-1.
template <class C>
struct HLoader {
  RowLoader<C::BM, C::BK, C::kThreads> rl;
  const uint16_t* H;
  int K, M, m0, tid;
  __device__ __forceinline__ void load(int k0) {
    rl.load([&](int i) {
      const int r = m0 + i < M ? m0 + i : M - 1;
      return H + static_cast<size_t>(r) * K;
    }, k0, tid);
  }
  __device__ __forceinline__ void store(uint16_t* lds, int ld) const { rl.store(lds, ld, tid); }
};

// B operand: W_out[K][Nc] is d-contiguous; each thread loads a 4(k) x 8(n)
// block and writes it transposed ([n][k]).  Consecutive lanes take
// consecutive k blocks, so the 8-byte LDS writes of a wavefront hit distinct
// banks.
template <class C>
struct WoutTransposeLoader {
  static constexpr int kBlocks = (C::BK / 4) * (C::BN / 8) / C::kThreads;
  static_assert((C::BK / 4) * (C::BN / 8) % C::kThreads == 0, "B tile must split evenly");
  uint4 rb[kBlocks][4];
  const uint16_t* W;
  int Nc, n0, tid;
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
      const int c = tid + i * C::kThreads;
      const int kb = c % (C::BK / 4);
      const int nb = c / (C::BK / 4);
      int col = n0 + nb * 8;
      col = col < Nc ? col : Nc - 8;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rb[i][r] = ldg16(W + static_cast<size_t>(k0 + kb * 4 + r) * Nc + col);
    }
  }
  __device__ __forceinline__ void store(uint16_t* Bs, int ld) const {
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
      const int c = tid + i * C::kThreads;
      const int kb = c % (C::BK / 4);
      const int nb = c / (C::BK / 4);
      // word q of row r holds columns 2q (low half) and 2q+1 (high half).
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint2 even = make_uint2(pack_lo(word(rb[i][0], q), word(rb[i][1], q)),
                                      pack_lo(word(rb[i][2], q), word(rb[i][3], q)));
        const uint2 odd = make_uint2(pack_hi(word(rb[i][0], q), word(rb[i][1], q)),
                                     pack_hi(word(rb[i][2], q), word(rb[i][3], q)));
        *reinterpret_cast<uint2*>(Bs + (nb * 8 + 2 * q) * ld + kb * 4) = even;
        *reinterpret_cast<uint2*>(Bs + (nb * 8 + 2 * q + 1) * ld + kb * 4) = odd;
      }
    }
  }
};

// y tile store from the transposed-block accumulators: lane holds y row
// (m-block i, lane % 32) and, for g = 0..3, the four consecutive columns
// 8g + 4*(lane/32) + 0..3 of n-block j -> one 8-byte store each.
template <class C>
__device__ __forceinline__ void store_y_tile(const f32x16_t (&acc)[C::kTm][C::kTn],
                                             uint16_t* __restrict__ y, int M, int Nc, int m0,
                                             int n0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = wave / C::kWavesN;
  const int wn = wave % C::kWavesN;
  const int row_base = m0 + wm * C::WM + (lane & 31);
#pragma unroll
  for (int i = 0; i < C::kTm; ++i) {
    const int row = row_base + i * 32;
    if (row >= M) continue;
    uint16_t* yrow = y + static_cast<size_t>(row) * Nc;
#pragma unroll
    for (int j = 0; j < C::kTn; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn * C::WN + j * 32 + g * 8 + (lane >> 5) * 4;
        if (col < Nc) {
          const uint2 v = make_uint2(pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                                     pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
          *reinterpret_cast<uint2*>(yrow + col) = v;
        }
      }
    }
  }
}

// The same tile stored through LDS: the accumulators go to a bf16 copy of
// the tile (rows padded by 16 bytes), then every thread writes 16-byte
// pieces with consecutive lanes along a row, so each store instruction
// writes whole 128-byte lines (the direct stores above write 16 bytes per
// row and line; measured on the OPT-1.3B-shaped projection they cost about
// a tenth of the kernel).  Needs Nc % 8 == 0 and a 16-byte aligned y.
template <class C>
constexpr int y_stage_pitch() { return C::BN * 2 + 16; }

template <class C>
constexpr size_t proj_lds_bytes() {
  constexpr size_t stage = size_t(C::BM) * y_stage_pitch<C>();
  return C::kLdsBytes > stage ? C::kLdsBytes : stage;
}

template <class C>
__device__ __forceinline__ void store_y_tile_lds(const f32x16_t (&acc)[C::kTm][C::kTn],
                                                 unsigned char* lds, uint16_t* __restrict__ y,
                                                 int M, int Nc, int m0, int n0) {
  constexpr int kPitch = y_stage_pitch<C>();
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = wave / C::kWavesN;
  const int wn = wave % C::kWavesN;
  // The main loop ended with a barrier: its stage buffers are free.
#pragma unroll
  for (int i = 0; i < C::kTm; ++i) {
    const int row = wm * C::WM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < C::kTn; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * C::WN + j * 32 + g * 8 + (lane >> 5) * 4;
        *reinterpret_cast<uint2*>(lds + row * kPitch + col * 2) =
            make_uint2(pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                       pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
      }
    }
  }
  __syncthreads();
  constexpr int kPieces = C::BN / 8;  // 16-byte pieces per row
  for (int e = threadIdx.x; e < C::BM * kPieces; e += C::kThreads) {
    const int r = e / kPieces;
    const int c = (e - r * kPieces) * 8;
    if (m0 + r < M && n0 + c < Nc)
      *reinterpret_cast<uint4*>(y + static_cast<size_t>(m0 + r) * Nc + n0 + c) =
          *reinterpret_cast<const uint4*>(lds + r * kPitch + c * 2);
  }
}

// y = H . W_out with both operands loaded straight into LDS by the
// multi-stage main loop: W_out in its own k-major layout (W_out[k][n]), whose
// fragments the main loop reads with transposing LDS reads, so W_out needs no
// preparation; H row-major, or K-blocked (HBLK: element (t, k) at
// ((k / 32) * M + t) * 32 + k % 32, as the H pass writes it inside the
// layer), where each stage's A tile is one contiguous block and every load
// fetches whole 128-byte lines.
template <class C, bool HBLK>
__global__ __launch_bounds__(C::kThreads) void proj_direct_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wout, uint16_t* __restrict__ y,
    int M, int K, int Nc, int tiles_n) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int tn = logical % tiles_n;
  const int tm = logical / tiles_n;
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;
  auto a_row = [&](int i) {
    const int r = m0 + i < M ? m0 + i : M - 1;
    return H + static_cast<size_t>(r) * (HBLK ? 32 : K);
  };
  const KMajorBOp<C> bop{KMajorB{Wout + n0, Nc, Nc - n0}};
  f32x16_t acc[C::kTm][C::kTn];
  gemm_mainloop_direct_op<C>(acc, lds, K, a_row, bop, HBLK ? static_cast<int64_t>(M) : 1);
  store_y_tile_lds<C>(acc, lds, y, M, Nc, m0, n0);
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void proj_mfma_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wout, uint16_t* __restrict__ y,
    int M, int K, int Nc, int tiles_m, int tiles_n) {
  extern __shared__ __align__(16) uint16_t smem[];
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int tn = logical % tiles_n;
  const int tm = logical / tiles_n;
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / C::kWavesN;
  const int wn = wave % C::kWavesN;

  HLoader<C> la;
  la.H = H;
  la.K = K;
  la.M = M;
  la.m0 = m0;
  la.tid = tid;
  WoutTransposeLoader<C> lb;
  lb.W = Wout;
  lb.Nc = Nc;
  lb.n0 = n0;
  lb.tid = tid;
  f32x16_t acc[C::kTm][C::kTn];
  gemm_mainloop<C>(acc, smem, K, la, lb);

  store_y_tile<C>(acc, y, M, Nc, m0, n0);
}

template <class C>
hipError_t launch_cfg(const Dims& s, const void* H, const void* Wout, void* y, hipStream_t st) {
  const int tiles_m = static_cast<int>((s.T + C::BM - 1) / C::BM);
  const int tiles_n = (s.d + C::BN - 1) / C::BN;
  auto kern = proj_mfma_kernel<C>;
  {
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void*>(kern), static_cast<int>(C::kLdsBytes));
    if (e != hipSuccess) return e;
  }
  kern<<<dim3(tiles_m * tiles_n), dim3(C::kThreads), C::kLdsBytes, st>>>(
      static_cast<const uint16_t*>(H), static_cast<const uint16_t*>(Wout),
      static_cast<uint16_t*>(y), static_cast<int>(s.T), static_cast<int>(s.K), s.d, tiles_m,
      tiles_n);
  return hipGetLastError();
}

using BigTile = TileCfg<256, 256, 64, 128, 128>;
using SmallTile = TileCfg<128, 128, 64, 64, 64>;
using BigDirect = DirectCfg<256, 256, 128, 64, 4>;
// Smaller products (the GPT-125M shape's 8192 x 768 output makes 96 big
// tiles): 256 x 128 or 128 x 128 tiles (the latter two workgroups per
// compute unit).
using WideDirect = DirectCfg<256, 128, 64, 64, 4>;
using MidDirect = DirectCfg<128, 128, 64, 64, 4>;

int64_t big_direct_tiles(const Dims& s) { return ((s.T + 255) / 256) * ((s.d + 255) / 256); }
int64_t mid_direct_tiles(const Dims& s) { return ((s.T + 127) / 128) * ((s.d + 127) / 128); }

// Output area the busiest compute unit computes with bm x bn tiles spread
// over the 256 units: the time model the tile choice minimises (ties go to
// the larger tile, which reuses each operand byte more).
int64_t cu_area(int64_t rows, int64_t cols, int bm, int bn) {
  const int64_t tiles = ((rows + bm - 1) / bm) * ((cols + bn - 1) / bn);
  return (tiles + 255) / 256 * bm * bn;
}

}  // namespace

bool project_mfma_supported(const Dims& s) {
  return s.dtype == 1 && s.K % 64 == 0 && s.d % 8 == 0 && s.d >= 8 && s.T >= 1;
}

hipError_t launch_project_mfma(const Dims& s, const void* H, const void* Wout, void* y,
                               hipStream_t st) {
  // Large products take 256x256 tiles; small ones 128x128 so the grid still
  // covers the 256 compute units.
  const int64_t big_tiles = ((s.T + 255) / 256) * ((s.d + 255) / 256);
  if (big_tiles >= 256) return launch_cfg<BigTile>(s, H, Wout, y, st);
  return launch_cfg<SmallTile>(s, H, Wout, y, st);
}

bool project_direct_supported(const Dims& s) {
  return project_mfma_supported(s) && s.K % 32 == 0 &&
         (big_direct_tiles(s) >= 256 || mid_direct_tiles(s) >= 256);
}

template <class C, bool HBLK>
hipError_t launch_direct_cfg(const Dims& s, const void* H, const void* Wout, void* y,
                             hipStream_t st) {
  const int tiles_m = static_cast<int>((s.T + C::BM - 1) / C::BM);
  const int tiles_n = (s.d + C::BN - 1) / C::BN;
  auto kern = proj_direct_kernel<C, HBLK>;
  constexpr size_t lds = proj_lds_bytes<C>();
  {
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void*>(kern), static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  kern<<<dim3(tiles_m * tiles_n), dim3(C::kThreads), lds, st>>>(
      static_cast<const uint16_t*>(H), static_cast<const uint16_t*>(Wout), static_cast<uint16_t*>(y),
      static_cast<int>(s.T), static_cast<int>(s.K), s.d, tiles_n);
  return hipGetLastError();
}

template <bool HBLK>
hipError_t launch_direct_pick(const Dims& s, const void* H, const void* Wout, void* y,
                              hipStream_t st) {
  const int64_t big = cu_area(s.T, s.d, 256, 256);
  const int64_t wide = cu_area(s.T, s.d, 256, 128);
  const int64_t mid = cu_area(s.T, s.d, 128, 128);
  if (big <= wide && big <= mid) return launch_direct_cfg<BigDirect, HBLK>(s, H, Wout, y, st);
  if (wide <= mid) return launch_direct_cfg<WideDirect, HBLK>(s, H, Wout, y, st);
  return launch_direct_cfg<MidDirect, HBLK>(s, H, Wout, y, st);
}

hipError_t launch_project_direct(const Dims& s, const void* H, const void* Wout, void* y,
                                 bool h_blocked, hipStream_t st) {
  if (h_blocked) return launch_direct_pick<true>(s, H, Wout, y, st);
  return launch_direct_pick<false>(s, H, Wout, y, st);
}

}  // namespace fff
