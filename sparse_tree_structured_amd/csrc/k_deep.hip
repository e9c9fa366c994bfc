// Deep tree levels of the FFF layer on gfx950, evaluated per token bucket.
//
// After the dense top-level product (k_route.hip) every (token, tree) sits at
// a node r of level k.  The deep levels k..D of that tree form the subtree
// rooted at r (2^(D-k+1) - 1 <= 15 nodes).  Only the nodes on the path are
// evaluated by the layer (explainer page, section 2), but tokens of one
// subtree share its weights, so:
//
//  bucket_count_kernel, bucket_scatter_kernel
//                 group, per (token chunk, tree), the chunk's tokens by
//                 their level-k node: within a wavefront, lanes with equal
//                 nodes find each other with one ballot per node bit, rank
//                 by a masked popcount and make one LDS atomic per
//                 (wavefront, bucket); the counts of a chunk's slices are
//                 scanned into offsets and token ids scattered into a
//                 permutation.
//
//  deep_kernel    one workgroup per (chunk, tree, subtree): copies the
//                 subtree's w_n and v_n rows (plus the v_n rows of the shared
//                 top path) straight into LDS once, then takes the bucket's
//                 tokens in groups of 16.  The eight waves split the model
//                 width of a group: each forms the partial logits of all
//                 subtree rows for the 16 tokens over its slice with
//                 v_mfma_f32_16x16x32_bf16, from x rows gathered straight
//                 from global memory (issued a group ahead); the partials are
//                 summed through LDS; every token is walked through the
//                 subtree and its finished slice
//                 H[t, p*h : (p+1)*h] = sum over all D+1 visited nodes of
//                 GELU(a) * v_n (GELU before the sum: section 3.C) is written
//                 with path_out.  The top-level terms use the logits recorded
//                 by the top-level kernel, so H is written exactly once.
//
// Tokens are bucketed per chunk, and the grid is ordered so that an XCD works
// through its chunks one at a time: the x rows a chunk gathers for all P
// trees are then reread from cache rather than HBM.  The chunk size trades
// that reuse against restaging every subtree's rows once per chunk
// (deep_chunk).
#include "common.hpp"
#include "launch.hpp"
#include "mfma_tile.hpp"

namespace fff {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSubRows = 16;  // subtree nodes per MFMA column block (15 used)

// Heap id of local node j of the subtree rooted at global node r.
__device__ __forceinline__ int64_t subtree_global(int64_t r, int j) {
  const int lvl = 31 - __clz(j + 1);  // floor(log2(j+1))
  return ((r + 1) << lvl) - 1 + (j - ((1 << lvl) - 1));
}

constexpr int kBucketThreads = 1024;
constexpr int kBucketMaxSlices = 16;  // slices per (chunk, tree)

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (uint64_t(1) << lane) - 1; }

// Lanes of this wavefront whose `valid` token has the same key (self
// included): one ballot per key bit, kept where the lane's own bit agrees.
__device__ __forceinline__ uint64_t same_key_lanes(bool valid, int key, int bits) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const bool on = (key >> b) & 1;
    const uint64_t m = __ballot(valid && on);
    peers &= on ? m : ~m;
  }
  return valid ? peers : 0;
}

// Each (token chunk, tree) is split into G slices of consecutive tokens, one
// workgroup per (chunk, tree, slice) in two launches, so that the grid covers
// the compute units even when chunks are few.  Per wavefront of 64 tokens,
// the lanes with equal level-k nodes find each other with k ballots; a lane's
// rank among them is a masked popcount, and their lowest lane makes the one
// LDS atomic of the (wavefront, bucket) pair.
//   bucket_count_kernel    counts its slice per bucket into cnt[chunk][tree][slice][S];
//   bucket_scatter_kernel  turns the counts of all slices of its (chunk, tree)
//                          into bucket offsets (written by slice 0) and its
//                          own slice's start in each bucket, and scatters its
//                          token ids there.
// Buckets keep each wavefront's tokens in order and the slices in slice
// order; wavefronts of one slice land in arbitrary order, and every token's
// result is independent of its neighbours in a bucket, so that order changes
// no output.
struct BucketSlice {
  int c, p, g, t0, t1;
};
__device__ __forceinline__ BucketSlice bucket_slice(int T, int P, int chunk, int G) {
  BucketSlice b;
  const int cp = blockIdx.x / G;
  b.g = blockIdx.x - cp * G;
  b.c = cp / P;
  b.p = cp - b.c * P;
  const int c0 = b.c * chunk;
  const int c1 = min(T, c0 + chunk);
  const int slice = (chunk + G - 1) / G;
  b.t0 = min(c1, c0 + b.g * slice);
  b.t1 = min(c1, b.t0 + slice);
  return b;
}

__global__ __launch_bounds__(kBucketThreads) void bucket_count_kernel(const int32_t* __restrict__ rec_next,
                                                                      int32_t* __restrict__ cnt_out,
                                                                      int T, int P, int k, int chunk,
                                                                      int G) {
  __shared__ int32_t cnt[256];
  const int S = 1 << k;  // k <= 8
  const BucketSlice b = bucket_slice(T, P, chunk, G);
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t* nx = rec_next + static_cast<int64_t>(b.p) * T;
  for (int i = threadIdx.x; i < S; i += kBucketThreads) cnt[i] = 0;
  __syncthreads();
  // The loop bound is uniform across the workgroup: every lane takes part
  // in the ballots, past the slice's end as an invalid lane.
  const int span = (b.t1 - b.t0 + kBucketThreads - 1) / kBucketThreads * kBucketThreads;
  for (int o = threadIdx.x; o < span; o += kBucketThreads) {
    const int t = b.t0 + o;
    const bool valid = t < b.t1;
    const int key = valid ? nx[t] - (S - 1) : 0;
    const uint64_t peers = same_key_lanes(valid, key, k);
    if (valid && lane == __ffsll(static_cast<unsigned long long>(peers)) - 1)
      atomicAdd(&cnt[key], __popcll(peers));
  }
  __syncthreads();
  int32_t* out = cnt_out + static_cast<int64_t>(blockIdx.x) * S;
  for (int i = threadIdx.x; i < S; i += kBucketThreads) out[i] = cnt[i];
}

__global__ __launch_bounds__(kBucketThreads) void bucket_scatter_kernel(const int32_t* __restrict__ rec_next,
                                                                        const int32_t* __restrict__ cnt_in,
                                                                        int32_t* __restrict__ perm,
                                                                        int32_t* __restrict__ offs, int T,
                                                                        int P, int k, int chunk, int G) {
  __shared__ int32_t tot[256];
  __shared__ int32_t cur[256];
  const int S = 1 << k;  // k <= 8
  const BucketSlice b = bucket_slice(T, P, chunk, G);
  const int lane = threadIdx.x & (kWave - 1);
  // Per bucket: the tokens of all slices, and those of the slices before this one.
  const int32_t* cin = cnt_in + static_cast<int64_t>(blockIdx.x - b.g) * S;
  for (int i = threadIdx.x; i < S; i += kBucketThreads) {
    int all = 0, before = 0;
    for (int g = 0; g < G; ++g) {
      const int v = cin[static_cast<int64_t>(g) * S + i];
      all += v;
      before += g < b.g ? v : 0;
    }
    tot[i] = all;
    cur[i] = before;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    // Exclusive scan of S <= 256 totals: four per lane, then across lanes.
    int v[4], sum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = lane * 4 + u;
      v[u] = i < S ? tot[i] : 0;
      sum += v[u];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int run = incl - sum;
    int32_t* ob = offs + (static_cast<int64_t>(b.c) * P + b.p) * (S + 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = lane * 4 + u;
      if (i < S) {
        if (b.g == 0) ob[i] = run;
        cur[i] += run;
      }
      run += v[u];
    }
    if (b.g == 0 && lane == kWave - 1) ob[S] = incl;
  }
  __syncthreads();
  const int32_t* nx = rec_next + static_cast<int64_t>(b.p) * T;
  int32_t* pp = perm + static_cast<int64_t>(b.p) * T + static_cast<int64_t>(b.c) * chunk;
  const int span = (b.t1 - b.t0 + kBucketThreads - 1) / kBucketThreads * kBucketThreads;
  for (int o = threadIdx.x; o < span; o += kBucketThreads) {
    const int t = b.t0 + o;
    const bool valid = t < b.t1;
    const int key = valid ? nx[t] - (S - 1) : 0;
    const uint64_t peers = same_key_lanes(valid, key, k);
    const int leader = valid ? __ffsll(static_cast<unsigned long long>(peers)) - 1 : lane;
    int base = 0;
    if (valid && lane == leader) base = atomicAdd(&cur[key], __popcll(peers));
    base = __shfl(base, leader);
    if (valid) pp[base + __popcll(peers & lanemask_lt(lane))] = t;
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS layout of deep_kernel (bytes, in order):
//   Wsub  kSubRows x (d + 8) bf16   subtree w_n rows (rows >= used are not
//                                   written; their products are never read)
//   Vsub  kSubRows x h bf16         subtree v_n rows
//   Vtop  k x h bf16                v_n rows of the top path shared by the bucket
//   part  kDeepWaves x 16 x 16 f32  per-wave partial logits [wave][row][token]
//   topl  16 x k f32                recorded top-level logits of a group's tokens
//   wgt   16 x 12 f32               v-row weights of a group's tokens (k + 4 <= 12)
//   bsub  kSubRows fp32             subtree biases
//   asub  kSubRows int32            1 = subtree node alive (static pruning)
constexpr int kDeepWaves = 8;
constexpr int kDeepSteps = 8;  // 32-wide k steps per wave: d <= 32 * 8 * 8
struct DeepLds {
  size_t w, vsub, vtop, part, topl, wgt, bsub, asub, total;
};
__host__ __device__ inline DeepLds deep_lds(int d, int h, int k) {
  DeepLds L;
  L.w = 0;
  L.vsub = L.w + size_t(kSubRows) * (d + 8) * 2;
  L.vtop = L.vsub + size_t(kSubRows) * h * 2;
  L.part = L.vtop + size_t(k) * h * 2;
  L.topl = L.part + size_t(kDeepWaves) * 16 * 16 * 4;
  L.wgt = L.topl + size_t(16) * k * 4;
  L.bsub = L.wgt + size_t(16) * 12 * 4;
  L.asub = L.bsub + kSubRows * 4;
  L.total = L.asub + kSubRows * 4;
  return L;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// Buffer loads: an offset past the buffer (kOob) returns zeros, so loads
// need no per-lane branch.
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not for its global loads still in flight (__syncthreads() would).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One workgroup per (chunk, tree p, level-k node s): the tokens of the
// bucket go through the subtree below s in groups of 16.  The subtree's w_n
// and v_n rows (and the v_n rows of the path above s) are copied straight
// into LDS once.  For a group, the eight waves split the model width: wave w
// loads its d/8 columns of the 16 token rows (one round of loads, issued a
// group ahead) and forms the partial logits of all 16 subtree rows with
// v_mfma_f32_16x16x32_bf16; the partials are summed in wave order through
// LDS.  Then wave w takes tokens 2w and 2w + 1, 32 lanes each: every lane
// walks its token through the subtree and forms h/32 consecutive columns of
//     H[t, p*h : (p+1)*h] = sum over all D+1 visited nodes of GELU(a) * v_n
// (GELU before the sum: explainer page, section 3.C; FFFpost applies it to
// the sum), the top levels' terms from the logits the top-level kernel
// recorded, so H is written exactly once; lane 0 writes path_out.
__global__ __launch_bounds__(kDeepWaves * 64, 2) void deep_kernel(
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
  const uint16_t* Wsub = reinterpret_cast<const uint16_t*>(lds + L.w);
  const uint16_t* Vsub = reinterpret_cast<const uint16_t*>(lds + L.vsub);
  const uint16_t* Vtop = reinterpret_cast<const uint16_t*>(lds + L.vtop);
  float* part = reinterpret_cast<float*>(lds + L.part);
  float* topl = reinterpret_cast<float*>(lds + L.topl);
  float* wgt = reinterpret_cast<float*>(lds + L.wgt);
  float* bsub = reinterpret_cast<float*>(lds + L.bsub);
  int32_t* asub = reinterpret_cast<int32_t*>(lds + L.asub);
  const int ld = d + 8;
  const uint16_t* Wp = W + static_cast<int64_t>(p) * N * d;
  const uint16_t* Vp = V + static_cast<int64_t>(p) * N * h;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;  // subtree row (A) / token of the group (B)
  const int q = lane >> 4;  // 8-wide k group within each 32-wide step
  const int tt = 2 * wave + (lane >> 5);  // token of the group this lane walks
  const int c32 = lane & 31;              // its h/32-column piece of H
  const int ngroups = (ntok + 15) / 16;
  const int nks = d / (32 * kDeepWaves);  // k steps of each wave's slice
  const int kw = wave * (d / kDeepWaves); // first column of the slice
  const __amdgpu_buffer_rsrc_t xbuf = buffer_of(x, uint32_t(T) * d * 2);
  const __amdgpu_buffer_rsrc_t lbuf = buffer_of(rec_logit, uint32_t(P) * T * k * 4);

  // Token id of lane m's row of group g (the last token past the bucket's
  // end: loads stay valid, results unused).
  auto tok_id = [&](int g) {
    const int i = g * 16 + m;
    return toks[i < ntok ? i : ntok - 1];
  };
  auto load_x = [&](uint4 (&xr)[kDeepSteps], int id) {
    const uint32_t base = uint32_t(id * d + kw + q * 8) * 2;
#pragma unroll
    for (int u = 0; u < kDeepSteps; ++u) xr[u] = buffer_load16(xbuf, u < nks ? base + u * 64 : kOob);
  };
  // Recorded logits of the top levels of a group's tokens (16 x k floats,
  // token-major like the record): element i = wave * 64 + lane of waves 0
  // and 1 (a zero elsewhere), written to LDS when the group is computed.
  const int ti = (wave * kWave + lane) / k;
  const bool top_lane = wave * kWave + lane < 16 * k;
  auto load_top = [&](int id) {
    const int tok = __shfl(id, ti < 16 ? ti : 15);
    const int i = wave * kWave + lane;
    return buffer_load_f32(
        lbuf, top_lane ? uint32_t((static_cast<int64_t>(p) * T + tok) * k + (i - ti * k)) * 4 : kOob);
  };

  // First group's loads, then the subtree's rows straight into LDS (1 KB
  // per wave-wide load, lane i at byte 16 i; all in flight together).
  int id0 = tok_id(0);
  int id1 = tok_id(ngroups > 1 ? 1 : 0);
  uint4 x0[kDeepSteps], x1[kDeepSteps];
  load_x(x0, id0);
  float tv0 = load_top(id0), tv1 = 0.0f;
  {
    const int row_bytes = d * 2;
    const int pieces = (row_bytes + 1023) >> 10;
    for (int i = wave; i < used * pieces; i += kDeepWaves) {
      const int j = i / pieces;
      const int pc = i - j * pieces;
      const int off = pc * 1024 + lane * 16;
      if (off < row_bytes)
        __builtin_amdgcn_global_load_lds(Wp + subtree_global(r, j) * d + (off >> 1),
                                         lds + L.w + size_t(j) * ld * 2 + pc * 1024, 16, 0, 0);
    }
    const int vrow = h * 2;  // <= 1 KB
    for (int i = wave; i < used + k; i += kDeepWaves) {
      int64_t n;
      size_t dst;
      if (i < used) {
        n = subtree_global(r, i);
        dst = L.vsub + size_t(i) * vrow;
      } else {
        const int l = i - used;      // top level l < k
        n = ((r + 1) >> (k - l)) - 1;  // ancestor of r at level l
        dst = L.vtop + size_t(l) * vrow;
      }
      if (lane * 16 < vrow)
        __builtin_amdgcn_global_load_lds(Vp + n * h + lane * 8, lds + dst, 16, 0, 0);
    }
  }
  if (tid < kSubRows) {
    const int j = tid;
    const int64_t g = static_cast<int64_t>(p) * N + (j < used ? subtree_global(r, j) : 0);
    const __amdgpu_buffer_rsrc_t abuf = buffer_of(alive ? static_cast<const void*>(alive) : x,
                                                  alive ? uint32_t(P * N) : 0);
    const uint16_t braw = b[g];
    const uint32_t al = __builtin_amdgcn_raw_buffer_load_b8(abuf, uint32_t(g), 0, 0);
    bsub[j] = j < used ? bf16_to_f32(braw) : 0.0f;
    asub[j] = j < used && (!alive || al != 0);
  }
  wait_vmcnt<0>();  // this wave's copies into LDS have landed
  lds_barrier();

  const uint16_t* wrow = Wsub + m * ld + kw + q * 8;
  const int hq = h / 32;
  // One group: partial logits of this wave's slice, their sum, the walk and
  // the token's H piece.
  auto compute = [&](int g, const uint4 (&xr)[kDeepSteps], float tv, int id) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kDeepSteps; ++u) {
      if (u < nks) {
        const uint4 wv = *reinterpret_cast<const uint4*>(wrow + u * 32);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv), as_bf16x8(xr[u]), acc, 0, 0,
                                                      0);
      }
    }
    // acc[rr] = this wave's part of row 4q + rr for token m.
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) part[(wave * 16 + 4 * q + rr) * 16 + m] = acc[rr];
    if (top_lane) topl[wave * kWave + lane] = tv;
    lds_barrier();
    const int idx = g * 16 + tt;
    const int tok = __shfl(id, tt);
    // Walk (every lane of the token: sums of the wave partials, no GELU).
    float av[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int jv[4];
    int j = 0;
#pragma unroll
    for (int lv = 0; lv < 4; ++lv) {
      if (lv < sub_levels) {
        float a = part[j * 16 + tt];
#pragma unroll
        for (int w = 1; w < kDeepWaves; ++w) a += part[(w * 16 + j) * 16 + tt];
        a += bsub[j];
        av[lv] = a;
        jv[lv] = j;
        if (lv + 1 < sub_levels) {
          int rr = go_right(a);
          if (!asub[2 * j + 1 + rr]) rr ^= 1;  // pruned child: its sibling
          j = 2 * j + 1 + rr;
        }
      }
    }
    // Weights of the token's D+1 v rows: lane l of its 32 forms level l's
    // (the recorded logit below level k, the walked one from k on) into LDS,
    // where the token's other lanes (same wavefront) read it: one GELU per
    // lane instead of one per level.
    float* wt = wgt + tt * 12;
    {
      float src;
      if (c32 < k) {
        src = topl[tt * k + c32];
      } else {
        const int lv = c32 - k;
        src = lv == 0 ? av[0] : lv == 1 ? av[1] : lv == 2 ? av[2] : av[3];
      }
      const float mine = post ? src : gelu_tanh(src);
      if (c32 < k + sub_levels) wt[c32] = mine;
    }
    if (idx < ntok) {
      uint16_t* out =
          H + static_cast<int64_t>(tok) * P * h + static_cast<int64_t>(p) * h + c32 * hq;
      for (int cc = 0; cc < hq; cc += 2) {
        float a0 = 0.0f, a1 = 0.0f;
        for (int l = 0; l < k; ++l) {
          const uint32_t v = *reinterpret_cast<const uint32_t*>(Vtop + l * h + c32 * hq + cc);
          const float w = wt[l];
          a0 += w * bf16lo(v);
          a1 += w * bf16hi(v);
        }
#pragma unroll
        for (int lv = 0; lv < 4; ++lv) {
          if (lv < sub_levels) {
            const uint32_t v =
                *reinterpret_cast<const uint32_t*>(Vsub + jv[lv] * h + c32 * hq + cc);
            const float w = wt[k + lv];
            a0 += w * bf16lo(v);
            a1 += w * bf16hi(v);
          }
        }
        if (post) {
          a0 = gelu_tanh(a0);
          a1 = gelu_tanh(a1);
        }
        *reinterpret_cast<uint32_t*>(out + cc) = pack_bf16x2(a0, a1);
      }
      if (c32 == 0 && path_out) {
        const int64_t leaf = subtree_global(r, jv[sub_levels - 1]);
        path_out[static_cast<int64_t>(tok) * P + p] =
            static_cast<int32_t>(leaf - ((int64_t(1) << D) - 1));
      }
    }
    lds_barrier();  // part is rewritten by the next group
  };

  // Groups in pairs over two register buffers; each group's loads are issued
  // one group ahead (past the last group they reload a valid token, unused).
  for (int g = 0; g < ngroups; g += 2) {
    load_x(x1, id1);
    tv1 = load_top(id1);
    const int id2 = tok_id(g + 2 < ngroups ? g + 2 : ngroups - 1);
    compute(g, x0, tv0, id0);
    if (g + 1 < ngroups) {
      load_x(x0, id2);
      tv0 = load_top(id2);
      const int id3 = tok_id(g + 3 < ngroups ? g + 3 : ngroups - 1);
      compute(g + 1, x1, tv1, id1);
      id0 = id2;
      id1 = id3;
    }
  }
}

}  // namespace

bool deep_supported(const Dims& s, int k) {
  // Each wave's slice of the width fits kDeepSteps k steps; V rows fit one
  // wave-wide copy and pair up per lane; byte offsets of x and of the
  // recorded logits fit the 32-bit buffer range.
  return s.dtype == 1 && k >= 1 && k <= 8 && k <= s.D && s.D - k + 1 <= 4 && s.d % 256 == 0 &&
         s.d <= 32 * kDeepWaves * kDeepSteps && s.h % 64 == 0 && s.h <= 512 &&
         deep_lds(s.d, s.h, k).total <= 80 * 1024 && s.T * int64_t(s.d) * 2 < (int64_t(1) << 31) &&
         int64_t(s.P) * s.T * k * 4 < (int64_t(1) << 31);
}

size_t deep_chunk(const Dims& s, int k) {
  // Tokens per chunk: about 32 MB of x rows, and at least 64 tokens per
  // level-k bucket on average so that the staged subtree rows serve several
  // 16-token groups.  Each chunk restages every subtree's rows, so small
  // chunks cost W_node traffic; large ones lose the x rows' cache reuse
  // across trees.  Measured at d = 2048, P = 32, h = 128, T = 16384 (ms per
  // forward, chunks of 2048 / 4096 / 8192 / 16384 tokens): D = 8: 0.83 /
  // 0.78 / 0.78 / 0.82; D = 9: 1.01 / 0.91 / 0.88 / 0.89; D = 10: 1.37 /
  // 1.16 / 1.07 / 1.05; D = 11: 2.06 / 1.65 / 1.45 / 1.36.
  int64_t c = (int64_t(32) << 20) / (int64_t(s.d) * 2);
  const int64_t per_bucket = int64_t(64) << k;
  c = c < per_bucket ? per_bucket : c;
  c = c < 64 ? 64 : c;
  return static_cast<size_t>(c < s.T ? c : s.T);
}

// Slices per (chunk, tree): about 512 workgroups in all, each slice at least
// one pass of a workgroup (kBucketThreads tokens), at most 16 slices.  With
// one workgroup per (chunk, tree) the two depth-8 and -11 headline shapes ran
// on 64 and 32 workgroups: 14 and 33 us.
int bucket_slices(const Dims& s, int chunk) {
  const int64_t groups = (s.T + chunk - 1) / chunk * s.P;
  int64_t g = (512 + groups - 1) / groups;
  const int64_t len = chunk < s.T ? chunk : s.T;
  const int64_t max_g = (len + kBucketThreads - 1) / kBucketThreads;
  g = g < max_g ? g : max_g;
  g = g < kBucketMaxSlices ? g : kBucketMaxSlices;
  return static_cast<int>(g < 1 ? 1 : g);
}

size_t bucket_count_bytes(const Dims& s, int k, int chunk) {
  const size_t nchunks = (size_t(s.T) + chunk - 1) / chunk;
  return nchunks * s.P * bucket_slices(s, chunk) * (size_t(1) << k) * sizeof(int32_t);
}

hipError_t launch_bucket(const Dims& s, int k, const int32_t* rec_next, int32_t* perm,
                         int32_t* offs, int32_t* cnt, int chunk, hipStream_t st) {
  const int nchunks = static_cast<int>((s.T + chunk - 1) / chunk);
  const int G = bucket_slices(s, chunk);
  const int64_t blocks = int64_t(nchunks) * s.P * G;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  bucket_count_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kBucketThreads), 0, st>>>(
      rec_next, cnt, static_cast<int>(s.T), s.P, k, chunk, G);
  bucket_scatter_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kBucketThreads), 0, st>>>(
      rec_next, cnt, perm, offs, static_cast<int>(s.T), s.P, k, chunk, G);
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
  auto kern = deep_kernel;
  {
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void*>(kern), 80 * 1024);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3(8 * per_xcd), dim3(kDeepWaves * 64), L.total, st>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W),
      static_cast<const uint16_t*>(b), static_cast<const uint16_t*>(V), rec_logit, perm, offs,
      static_cast<uint16_t*>(H), path_out, static_cast<int>(s.T), s.d, s.P, s.D, s.h, s.N, k,
      chunk, nchunks, s.variant, s.prune ? s.prune->alive : nullptr);
  return hipGetLastError();
}

}  // namespace fff
