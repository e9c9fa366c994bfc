// Deep tree levels of the FFF layer on gfx950, evaluated per token bucket.
//
// After the dense top-level product (k_route.hip) every (token, tree) sits at
// a node r of level k.  The deep levels k..D of that tree form the subtree
// rooted at r (2^(D-k+1) - 1 <= 15 nodes).  Only the nodes on the path are
// evaluated by the layer (explainer page, section 2), but tokens of one
// subtree share its weights, so:
//
//  bucket_kernel  groups, per (token chunk, tree), the chunk's tokens by
//                 their level-k node: a wavefront matches equal buckets with
//                 ballots, ranks lanes with a masked popcount, and makes one
//                 LDS atomic per (wavefront, bucket); counts are scanned into
//                 offsets and token ids scattered into a permutation.
//
//  deep_kernel    one workgroup per (chunk, tree, subtree): stages the
//                 subtree's w_n rows, biases and v_n rows (plus the v_n rows
//                 of the shared top path) in LDS once, then for groups of 16
//                 tokens computes all subtree logits with
//                 v_mfma_f32_16x16x32_bf16 over x rows gathered straight from
//                 global memory, walks the subtree in registers (cross-lane
//                 shuffles), and writes the token's finished slice
//                 H[t, p*h : (p+1)*h] = sum over all D+1 visited nodes of
//                 GELU(a) * v_n (GELU before the sum: section 3.C), together
//                 with path_out.  The top-level terms use the logits recorded
//                 by the top-level kernel, so H is written exactly once.
//
// Chunks are sized to fit an XCD's L2 and the grid is ordered so each XCD
// works through its own chunks one at a time: the x rows a chunk gathers for
// all P trees stay in that XCD's L2.
#include "common.hpp"
#include "launch.hpp"
#include "mfma_tile.hpp"

namespace fff {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte load that should not displace reused data in L2.
__device__ __forceinline__ uint4 ldg16_stream(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

constexpr int kSubRows = 16;  // subtree nodes per MFMA column block (15 used)

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return (uint64_t(1) << lane) - 1;
}

// Heap id of local node j of the subtree rooted at global node r.
__device__ __forceinline__ int64_t subtree_global(int64_t r, int j) {
  const int lvl = 31 - __clz(j + 1);  // floor(log2(j+1))
  return ((r + 1) << lvl) - 1 + (j - ((1 << lvl) - 1));
}

__global__ __launch_bounds__(256) void bucket_kernel(const int32_t* __restrict__ rec_next,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ offs, int T, int P,
                                                     int k, int chunk) {
  extern __shared__ int32_t sh[];  // cnt[S], cur[S]
  const int S = 1 << k;
  int32_t* cnt = sh;
  int32_t* cur = sh + S;
  const int c = blockIdx.x / P;
  const int p = blockIdx.x - c * P;
  const int t0 = c * chunk;
  const int t1 = min(T, t0 + chunk);
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t* nx = rec_next + static_cast<int64_t>(p) * T;
  for (int i = threadIdx.x; i < S; i += blockDim.x) cnt[i] = 0;
  __syncthreads();

  // Pass 1: counts.  Pass 2: positions.  Both walk the chunk in the same
  // order with the same wavefront matching.
  for (int pass = 0; pass < 2; ++pass) {
    int32_t* ctr = pass == 0 ? cnt : cur;
    for (int base = t0; base < t1; base += blockDim.x) {
      const int t = base + threadIdx.x;
      const bool valid = t < t1;
      const int s = valid ? nx[t] - (S - 1) : -1;
      uint64_t active = __ballot(valid);
      int pos = 0;
      while (active) {
        const int leader = __ffsll(static_cast<unsigned long long>(active)) - 1;
        const int ls = __shfl(s, leader);
        const uint64_t mask = __ballot(valid && s == ls);
        int got = 0;
        if (lane == leader) got = atomicAdd(&ctr[ls], __popcll(mask));
        got = __shfl(got, leader);
        if (valid && s == ls) pos = got + __popcll(mask & lanemask_lt(lane));
        active &= ~mask;
      }
      if (pass == 1 && valid) perm[static_cast<int64_t>(p) * T + t0 + pos] = t;
    }
    __syncthreads();
    if (pass == 0) {
      if (threadIdx.x == 0) {
        int32_t* o = offs + (static_cast<int64_t>(c) * P + p) * (S + 1);
        int run = 0;
        for (int i = 0; i < S; ++i) {
          o[i] = run;
          cur[i] = run;
          run += cnt[i];
        }
        o[S] = run;
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS layout of deep_kernel (bytes, in order):
//   Wsub  kSubRows x (d + 8) bf16   subtree w_n rows (rows >= used are zero)
//   Vsub  kSubRows x h bf16         subtree v_n rows
//   Vtop  k x h bf16                v_n rows of the top path shared by the bucket
//   bsub  kSubRows fp32             subtree biases
//   asub  kSubRows int32            1 = subtree node alive (static pruning)
struct DeepLds {
  size_t w, vsub, vtop, bsub, asub, total;
};
__host__ __device__ inline DeepLds deep_lds(int d, int h, int k) {
  DeepLds L;
  L.w = 0;
  L.vsub = L.w + size_t(kSubRows) * (d + 8) * 2;
  L.vtop = L.vsub + size_t(kSubRows) * h * 2;
  L.bsub = L.vtop + size_t(k) * h * 2;
  L.asub = L.bsub + kSubRows * 4;
  L.total = L.asub + kSubRows * 4;
  return L;
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64, 2) void deep_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, const uint16_t* __restrict__ b,
    const uint16_t* __restrict__ V, const float* __restrict__ rec_logit,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offs, uint16_t* __restrict__ H,
    int32_t* __restrict__ path_out, int T, int d, int P, int D, int h, int64_t N, int k,
    int chunk, int nchunks, int post, const uint8_t* __restrict__ alive) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int S = 1 << k;
  const int ipc = P * S;  // items per chunk
  // Hardware sends workgroup b to XCD b % 8.  With at least 8 chunks each
  // XCD works through its own chunks (c % 8 == XCD) one at a time; with
  // fewer, chunk c is shared by the XCDs x with x % nchunks == c, which take
  // its items in turn, so that no XCD idles.
  const int bid = blockIdx.x;
  const int xcd = bid % 8;
  const int local = bid / 8;
  int c, item;
  if (nchunks >= 8) {
    c = (local / ipc) * 8 + xcd;
    item = local % ipc;
  } else {
    c = xcd % nchunks;
    const int share = (8 - 1 - c) / nchunks + 1;  // XCDs on chunk c
    item = local * share + xcd / nchunks;
  }
  if (c >= nchunks || item >= ipc) return;
  const int p = item / S;
  const int s = item - p * S;
  const int32_t* o = offs + (static_cast<int64_t>(c) * P + p) * (S + 1);
  const int beg = o[s];
  const int ntok = o[s + 1] - beg;
  if (ntok <= 0) return;
  const int32_t* toks = perm + static_cast<int64_t>(p) * T + static_cast<int64_t>(c) * chunk + beg;

  const int sub_levels = D - k + 1;             // levels in the subtree
  const int used = (1 << sub_levels) - 1;       // subtree nodes
  const int64_t r = (int64_t(1) << k) - 1 + s;  // subtree root (heap id)
  const DeepLds L = deep_lds(d, h, k);
  uint16_t* Wsub = reinterpret_cast<uint16_t*>(lds + L.w);
  uint16_t* Vsub = reinterpret_cast<uint16_t*>(lds + L.vsub);
  uint16_t* Vtop = reinterpret_cast<uint16_t*>(lds + L.vtop);
  float* bsub = reinterpret_cast<float*>(lds + L.bsub);
  int32_t* asub = reinterpret_cast<int32_t*>(lds + L.asub);
  const int ld = d + 8;
  const uint16_t* Wp = W + static_cast<int64_t>(p) * N * d;
  const uint16_t* Vp = V + static_cast<int64_t>(p) * N * h;

  // Stage the subtree (and the top path's v rows) once.
  const int wchunks = d / 8;
  for (int e = threadIdx.x; e < kSubRows * wchunks; e += blockDim.x) {
    const int j = e / wchunks;
    const int cc = e - j * wchunks;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < used) v = ldg16_stream(Wp + subtree_global(r, j) * d + cc * 8);
    *reinterpret_cast<uint4*>(Wsub + j * ld + cc * 8) = v;
  }
  const int hchunks = h / 8;
  for (int e = threadIdx.x; e < (kSubRows + k) * hchunks; e += blockDim.x) {
    const int j = e / hchunks;
    const int cc = e - j * hchunks;
    if (j < kSubRows) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < used) v = ldg16(Vp + subtree_global(r, j) * h + cc * 8);
      *reinterpret_cast<uint4*>(Vsub + j * h + cc * 8) = v;
    } else {
      const int l = j - kSubRows;                   // top level l < k
      const int64_t n = ((r + 1) >> (k - l)) - 1;  // ancestor of r at level l
      *reinterpret_cast<uint4*>(Vtop + l * h + cc * 8) = ldg16(Vp + n * h + cc * 8);
    }
  }
  for (int j = threadIdx.x; j < kSubRows; j += blockDim.x) {
    const int64_t g = static_cast<int64_t>(p) * N + (j < used ? subtree_global(r, j) : 0);
    bsub[j] = j < used ? bf16_to_f32(b[g]) : 0.0f;
    asub[j] = j < used && (!alive || alive[g]);
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m = lane & 15;  // token within the group (and subtree node row for W)
  const int q = lane >> 4;  // k sub-block of the operands; h quarter of the output
  const int ngroups = (ntok + 15) / 16;
  const int my_groups = wave < ngroups ? (ngroups - wave + WAVES - 1) / WAVES : 0;
  const int nb = d / 256;  // batches of 4 k-steps (64 k each) per token group
  const int total = my_groups * nb;
  const uint16_t* wrow = Wsub + m * ld + q * 16;
  const int hq = h / 4;  // outputs per lane

  // x rows are read with 32 contiguous bytes per lane (k = 64 s + 16 q + 0..15;
  // the four lanes of a token cover one 128-byte line per step), double
  // buffered one batch (4 steps, 8 loads) ahead, across group boundaries.
  auto tok_of = [&](int i) {  // token id of this lane's row in the wave's i-th group
    const int idx = (wave + WAVES * i) * 16 + m;
    return toks[idx < ntok ? idx : ntok - 1];
  };
  int issue_tok = total > 0 ? tok_of(0) : 0;
  auto issue = [&](uint4 (&xa)[4], uint4 (&xb)[4], int f) {
    const int i = f / nb;
    const int bb = f - i * nb;
    if (bb == 0 && i > 0) issue_tok = tok_of(i);
    const uint16_t* xr = x + static_cast<int64_t>(issue_tok) * d + q * 16 + bb * 256;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xa[u] = ldg16(xr + u * 64);
      xb[u] = ldg16(xr + u * 64 + 8);
    }
  };

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto finish = [&](int i) {
    const int idx = (wave + WAVES * i) * 16 + m;
    const bool valid = idx < ntok;
    const int tok = toks[valid ? idx : ntok - 1];
    // Walk the subtree.  Node j of token m lives in lane m + 16*(j/4), register j%4.
    float gv[kSubRows / 4 + 1];
    int jv[kSubRows / 4 + 1];
    int j = 0;
    for (int lv = 0; lv < sub_levels; ++lv) {
      const int src = m + 16 * (j >> 2);
      const float v0 = __shfl(acc[0], src);
      const float v1 = __shfl(acc[1], src);
      const float v2 = __shfl(acc[2], src);
      const float v3 = __shfl(acc[3], src);
      const int rr = j & 3;
      const float a = (rr == 0 ? v0 : rr == 1 ? v1 : rr == 2 ? v2 : v3) + bsub[j];
      gv[lv] = post ? a : gelu_tanh(a);
      jv[lv] = j;
      if (lv + 1 < sub_levels) {
        int rr2 = go_right(a);
        if (!asub[2 * j + 1 + rr2]) rr2 ^= 1;  // pruned child: its sibling
        j = 2 * j + 1 + rr2;
      }
    }
    if (!valid) return;
    // H slice of this lane: columns [q*hq, (q+1)*hq) of tree p.
    const float* tl = rec_logit + (static_cast<int64_t>(p) * T + tok) * k;
    float gt[8];
    for (int l = 0; l < k; ++l) gt[l] = post ? tl[l] : gelu_tanh(tl[l]);
    uint16_t* out = H + static_cast<int64_t>(tok) * P * h + static_cast<int64_t>(p) * h + q * hq;
    for (int c8 = 0; c8 < hq; c8 += 8) {
      float a8[8] = {};
      for (int l = 0; l < k; ++l) {
        const uint4 v = *reinterpret_cast<const uint4*>(Vtop + l * h + q * hq + c8);
        const float gg = gt[l];
        a8[0] += gg * bf16lo(v.x); a8[1] += gg * bf16hi(v.x);
        a8[2] += gg * bf16lo(v.y); a8[3] += gg * bf16hi(v.y);
        a8[4] += gg * bf16lo(v.z); a8[5] += gg * bf16hi(v.z);
        a8[6] += gg * bf16lo(v.w); a8[7] += gg * bf16hi(v.w);
      }
      for (int lv = 0; lv < sub_levels; ++lv) {
        const uint4 v = *reinterpret_cast<const uint4*>(Vsub + jv[lv] * h + q * hq + c8);
        const float gg = gv[lv];
        a8[0] += gg * bf16lo(v.x); a8[1] += gg * bf16hi(v.x);
        a8[2] += gg * bf16lo(v.y); a8[3] += gg * bf16hi(v.y);
        a8[4] += gg * bf16lo(v.z); a8[5] += gg * bf16hi(v.z);
        a8[6] += gg * bf16lo(v.w); a8[7] += gg * bf16hi(v.w);
      }
      if (post) {
#pragma unroll
        for (int u = 0; u < 8; ++u) a8[u] = gelu_tanh(a8[u]);
      }
      const u32x4_t packed = {pack_bf16x2(a8[0], a8[1]), pack_bf16x2(a8[2], a8[3]),
                              pack_bf16x2(a8[4], a8[5]), pack_bf16x2(a8[6], a8[7])};
      __builtin_nontemporal_store(packed, reinterpret_cast<u32x4_t*>(out + c8));
    }
    if (q == 0 && path_out) {
      const int64_t leaf = subtree_global(r, jv[sub_levels - 1]);
      path_out[static_cast<int64_t>(tok) * P + p] =
          static_cast<int32_t>(leaf - ((int64_t(1) << D) - 1));
    }
  };
  auto consume = [&](const uint4 (&xa)[4], const uint4 (&xb)[4], int f) {
    const int i = f / nb;
    const int bb = f - i * nb;
    if (bb == 0) acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t* w = wrow + bb * 256;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 wa = *reinterpret_cast<const uint4*>(w + u * 64);
      const uint4 wb = *reinterpret_cast<const uint4*>(w + u * 64 + 8);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa), as_bf16x8(xa[u]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wb), as_bf16x8(xb[u]), acc, 0, 0, 0);
    }
    if (bb == nb - 1) finish(i);
  };

  uint4 xa0[4], xb0[4], xa1[4], xb1[4];
  if (total > 0) issue(xa0, xb0, 0);
  for (int f = 0; f < total; f += 2) {
    if (f + 1 < total) issue(xa1, xb1, f + 1);
    consume(xa0, xb0, f);
    if (f + 1 < total) {
      if (f + 2 < total) issue(xa0, xb0, f + 2);
      consume(xa1, xb1, f + 1);
    }
  }
}

}  // namespace

bool deep_supported(const Dims& s, int k) {
  return s.dtype == 1 && k >= 1 && k <= 8 && k <= s.D && s.D - k + 1 <= 4 && s.d % 256 == 0 &&
         s.h % 32 == 0 && deep_lds(s.d, s.h, k).total <= 80 * 1024;
}

size_t deep_chunk(const Dims& s, int k) {
  // Tokens per chunk: about 16 MB of x rows, and at least 32 tokens per
  // level-k bucket on average so that the staged subtree rows serve whole
  // 16-token groups.  Each chunk restages every subtree's rows, so small
  // chunks cost W_node traffic; large ones lose the x rows' cache reuse
  // across trees.  Measured at d = 2048, P = 32, h = 128, T = 16384 (ms per
  // forward, chunks of 1024 / 2048 / 4096 / 8192 / 16384 tokens): D = 8:
  // 1.09 / 0.98 / 1.00 / 1.05 / 1.28; D = 9: 1.79 / 1.25 / 1.16 / 1.27 / 1.54;
  // D = 10: 3.17 / 2.04 / 1.55 / 1.54 / 1.89; D = 11: 5.99 / 3.62 / 2.51 /
  // 2.09 / 2.35.
  int64_t c = (16 << 20) / (int64_t(s.d) * 2);
  const int64_t per_bucket = int64_t(32) << k;
  c = c < per_bucket ? per_bucket : c;
  c = c < 64 ? 64 : c;
  return static_cast<size_t>(c < s.T ? c : s.T);
}

hipError_t launch_bucket(const Dims& s, int k, const int32_t* rec_next, int32_t* perm,
                         int32_t* offs, int chunk, hipStream_t st) {
  const int nchunks = static_cast<int>((s.T + chunk - 1) / chunk);
  const size_t lds = 2 * sizeof(int32_t) * (size_t(1) << k);
  bucket_kernel<<<dim3(nchunks * s.P), dim3(256), lds, st>>>(rec_next, perm, offs,
                                                             static_cast<int>(s.T), s.P, k, chunk);
  return hipGetLastError();
}

hipError_t launch_deep(const Dims& s, int k, const void* x, const void* W, const void* b,
                       const void* V, const float* rec_logit, const int32_t* perm,
                       const int32_t* offs, void* H, int32_t* path_out, int chunk,
                       hipStream_t st) {
  const int nchunks = static_cast<int>((s.T + chunk - 1) / chunk);
  const int ipc = s.P << k;
  // Workgroups per XCD: every chunk's items (at least 8 chunks), or the
  // items of a chunk split over the fewest XCDs that share one.
  const int per_xcd = nchunks >= 8 ? ((nchunks + 7) / 8) * ipc
                                   : (ipc + 8 / nchunks - 1) / (8 / nchunks);
  const DeepLds L = deep_lds(s.d, s.h, k);
  auto kern = deep_kernel<8>;
  {
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void*>(kern), 80 * 1024);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3(8 * per_xcd), dim3(8 * 64), L.total, st>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W),
      static_cast<const uint16_t*>(b), static_cast<const uint16_t*>(V), rec_logit, perm, offs,
      static_cast<uint16_t*>(H), path_out, static_cast<int>(s.T), s.d, s.P, s.D, s.h, s.N, k,
      chunk, nchunks, s.variant, s.prune ? s.prune->alive : nullptr);
  return hipGetLastError();
}

}  // namespace fff
