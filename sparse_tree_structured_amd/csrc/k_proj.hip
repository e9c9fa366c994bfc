// Output projection of the FFF layer on gfx950 matrix cores.
//
// The tree outputs are concatenated and passed through one final linear
// projection (paper page, Figure 1(c) caption): y[T,d] = H[T,K] . W_out[K,d]
// with K = P*h.  bf16 operands, fp32 accumulation (v_mfma_f32_32x32x16_bf16),
// bf16 result rounded to nearest even.
//
// Tiling: a workgroup owns a BM x BN tile of y; each wavefront a WM x WN
// sub-tile made of 32x32 MFMA blocks.  K advances in steps of BK through two
// LDS buffers (global loads for step k+1 are issued before the matrix-core
// work of step k).  H rows are K-contiguous and go to LDS as they are.
// W_out rows are d-contiguous, but a matrix-core operand lane needs 8
// consecutive K values of one column, so each thread loads a 4(K) x 8(d)
// block, transposes it in registers with byte permutes and writes it to LDS
// column-major ([n][k]).
//
// Workgroups are spread round-robin over the 8 XCDs; the tile order is
// remapped so that the tiles one XCD runs at the same time share rows of H
// and columns of W_out in that XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace fff {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct U4 {
  uint32_t v[4];
};

__device__ __forceinline__ U4 ldg16(const uint16_t* p) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  U4 r;
  r.v[0] = q.x;
  r.v[1] = q.y;
  r.v[2] = q.z;
  r.v[3] = q.w;
  return r;
}

// Select the low (or high) 16-bit halves of two dwords into one dword:
// result = (b.half << 16) | a.half.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int BM, int BN, int BK, int WM, int WN>
struct ProjCfg {
  static constexpr int kWavesM = BM / WM;
  static constexpr int kWavesN = BN / WN;
  static constexpr int kThreads = kWavesM * kWavesN * kWave;
  static constexpr int kLd = BK + 8;  // LDS row pitch in elements (16-byte pad)
  static constexpr int kAChunks = BM * BK / 8 / kThreads;        // 16-byte loads of H
  static constexpr int kBBlocks = (BK / 4) * (BN / 8) / kThreads;  // 4x8 blocks of W_out
  static constexpr int kTm = WM / 32;
  static constexpr int kTn = WN / 32;
  static constexpr int kStage = (BM + BN) * kLd;  // elements per LDS buffer
  static_assert(BM * BK / 8 % kThreads == 0, "A tile must split evenly");
  static_assert((BK / 4) * (BN / 8) % kThreads == 0, "B tile must split evenly");
  static_assert(BK % 16 == 0 && WM % 32 == 0 && WN % 32 == 0, "MFMA block shape");
};

template <int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void proj_mfma_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wout, uint16_t* __restrict__ y,
    int M, int K, int Nc, int tiles_m, int tiles_n) {
  using C = ProjCfg<BM, BN, BK, WM, WN>;
  extern __shared__ __align__(16) uint16_t smem[];

  // XCD-aware tile order: hardware sends workgroup b to XCD b % 8.  Give
  // each XCD a contiguous range of row panels (all column tiles of each), so
  // H is fetched from HBM once in total and W_out once per XCD, and the
  // tiles an XCD runs together share W_out's k-slices in its L2.
  const int nblk = gridDim.x;
  const int b = blockIdx.x;
  int logical = (b % 8) * (nblk / 8) + (b / 8);
  if ((nblk % 8) != 0) logical = b;  // uneven grids keep the plain order
  const int tn = logical % tiles_n;
  const int tm = logical / tiles_n;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / C::kWavesN;
  const int wn = wave % C::kWavesN;

  U4 ra[C::kAChunks];
  U4 rb[C::kBBlocks][4];

  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::kAChunks; ++i) {
      const int c = tid + i * C::kThreads;
      const int row = c / (BK / 8);
      const int kc = c % (BK / 8);
      int r = m0 + row;
      r = r < M ? r : M - 1;
      ra[i] = ldg16(H + static_cast<size_t>(r) * K + k0 + kc * 8);
    }
#pragma unroll
    for (int i = 0; i < C::kBBlocks; ++i) {
      const int c = tid + i * C::kThreads;
      const int nb = c % (BN / 8);
      const int kb = c / (BN / 8);
      int col = n0 + nb * 8;
      col = col < Nc ? col : Nc - 8;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rb[i][r] = ldg16(Wout + static_cast<size_t>(k0 + kb * 4 + r) * Nc + col);
    }
  };

  auto store_lds = [&](int buf) {
    uint16_t* As = smem + buf * C::kStage;
    uint16_t* Bs = As + BM * C::kLd;
#pragma unroll
    for (int i = 0; i < C::kAChunks; ++i) {
      const int c = tid + i * C::kThreads;
      const int row = c / (BK / 8);
      const int kc = c % (BK / 8);
      *reinterpret_cast<uint4*>(As + row * C::kLd + kc * 8) =
          make_uint4(ra[i].v[0], ra[i].v[1], ra[i].v[2], ra[i].v[3]);
    }
#pragma unroll
    for (int i = 0; i < C::kBBlocks; ++i) {
      const int c = tid + i * C::kThreads;
      const int nb = c % (BN / 8);
      const int kb = c / (BN / 8);
      // rb[i][r].v[q] holds columns 2q (low half) and 2q+1 (high half) of row r.
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint2 even = make_uint2(pack_lo(rb[i][0].v[q], rb[i][1].v[q]),
                                      pack_lo(rb[i][2].v[q], rb[i][3].v[q]));
        const uint2 odd = make_uint2(pack_hi(rb[i][0].v[q], rb[i][1].v[q]),
                                     pack_hi(rb[i][2].v[q], rb[i][3].v[q]));
        *reinterpret_cast<uint2*>(Bs + (nb * 8 + 2 * q) * C::kLd + kb * 4) = even;
        *reinterpret_cast<uint2*>(Bs + (nb * 8 + 2 * q + 1) * C::kLd + kb * 4) = odd;
      }
    }
  };

  f32x16_t acc[C::kTm][C::kTn];
#pragma unroll
  for (int i = 0; i < C::kTm; ++i)
#pragma unroll
    for (int j = 0; j < C::kTn; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int ksteps = K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < ksteps) load_global((ks + 1) * BK);
    const uint16_t* As = smem + cur * C::kStage;
    const uint16_t* Bs = As + BM * C::kLd;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8_t af[C::kTm], bfr[C::kTn];
#pragma unroll
      for (int i = 0; i < C::kTm; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * WM + i * 32 + lrow) * C::kLd + kk + lk);
#pragma unroll
      for (int j = 0; j < C::kTn; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * WN + j * 32 + lrow) * C::kLd + kk + lk);
#pragma unroll
      for (int i = 0; i < C::kTm; ++i)
#pragma unroll
        for (int j = 0; j < C::kTn; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < ksteps) store_lds(cur ^ 1);
    __syncthreads();
  }

  // Accumulator layout of a 32x32 block: lane holds column (lane % 32) and
  // rows 8*(r/4) + 4*(lane/32) + (r%4) for r = 0..15.
#pragma unroll
  for (int i = 0; i < C::kTm; ++i)
#pragma unroll
    for (int j = 0; j < C::kTn; ++j) {
      const int col = n0 + wn * WN + j * 32 + lrow;
      if (col >= Nc) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < M) y[static_cast<size_t>(row) * Nc + col] = f32_to_bf16(acc[i][j][r]);
      }
    }
}

constexpr int kBM = 128, kBN = 128, kBK = 64, kWM = 64, kWN = 64;
using Cfg = ProjCfg<kBM, kBN, kBK, kWM, kWN>;

}  // namespace

bool project_mfma_supported(const Dims& s) {
  return s.dtype == 1 && s.K % kBK == 0 && s.d % 8 == 0 && s.d >= 8 && s.T >= 1;
}

hipError_t launch_project_mfma(const Dims& s, const void* H, const void* Wout, void* y,
                               hipStream_t st) {
  const int tiles_m = static_cast<int>((s.T + kBM - 1) / kBM);
  const int tiles_n = (s.d + kBN - 1) / kBN;
  const size_t lds = 2 * Cfg::kStage * sizeof(uint16_t);
  auto kern = proj_mfma_kernel<kBM, kBN, kBK, kWM, kWN>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  kern<<<dim3(tiles_m * tiles_n), dim3(Cfg::kThreads), lds, st>>>(
      static_cast<const uint16_t*>(H), static_cast<const uint16_t*>(Wout),
      static_cast<uint16_t*>(y), static_cast<int>(s.T), static_cast<int>(s.K), s.d, tiles_m,
      tiles_n);
  return hipGetLastError();
}

}  // namespace fff
