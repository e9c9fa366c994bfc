// Deep tree levels of the FFF layer on gfx950, one token tile at a time.
//
// Only the nodes on a token's path are evaluated by the layer (explainer
// page, gist.science, section 2, Methodology).  After the dense product over
// the top levels 0..k-1 (k_route.hip) every (token, tree) sits at one of the
// S = 2^k nodes of level k; the levels k..D below it form a subtree of at
// most 15 nodes.  subtree_kernel evaluates, for every token of a tile and
// every tree of a tree group, the 16-column block of its own subtree only:
//
//   one workgroup = M tokens x G trees.  Per K step of 32, the tile's x rows
//   (M x 64 bytes) and the G trees' subtree rows (G x S x 16 rows) go
//   straight into LDS (global_load_lds, two stages), so x is read once per
//   tree group instead of once per tree.  Before the main loop the tile's
//   tokens are grouped, per tree, by their level-k node: units of 32 tokens
//   that share a subtree (the last one of a subtree padded), each unit two
//   groups of 16.  A group is one v_mfma_f32_16x16x32_bf16 per K step: its
//   16 x rows, read from LDS through the group's row list (the permutation
//   costs nothing there), against the 16 rows of its subtree, which are read
//   once per unit for both of its groups.  Whole units are split evenly over
//   the eight waves.
//
// The epilogue walks each token through its subtree (a = logit + b_n; left
// iff a < 0; NaN and zeros right) and records the logits of levels k..D in
// rec_logit[p][t][k..D] (stride D+1, beside the top levels' logits) and the
// leaf in rec_next[p][t]; hbuild_kernel then forms H and path_out from the
// complete records.
//
// Within a subtree the order of a group's tokens is free (every token's
// result is its own).  Tokens are ordered by (rank within their class,
// class), the class being the low three bits of the token's row, so that
// each eight consecutive rows of a group take distinct classes where the
// counts allow: the operand read, which the LDS serves eight lanes at a
// time, is then free of bank conflicts under the rows' XOR swizzle (chunk c
// of row r at slot c ^ ((r >> 1) & 3), a function of row bits 0-2 together
// with the row's bank offset; with bits 2-3, as the 32 x 32 x 16 products
// use, every such read measured 2-way conflicts).
#include "common.hpp"
#include "launch.hpp"
#include "mfma_tile.hpp"

namespace fff {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Chunk swizzle of the staged rows: chunk c of row r at slot c ^ ((r >> 1) & 3),
// conflict-free for the 16-row operand fetches below when the 16 rows differ
// in their low four bits.
constexpr int kSwz = 1;

// Token classes for the operand-read order: row bits 0-2 (the bits the
// swizzle above and the row's bank offset depend on).  A 16 x 16 x 32
// operand read is served eight lanes (eight rows) at a time, so eight rows
// with distinct classes read without bank conflicts.
constexpr int kClasses = 8;
// Tokens per subtree are padded to whole units of kUnit = 16 * kPair tokens;
// the kPair groups of a unit share their subtree, so one read of its node
// rows serves kPair matrix-core products.
constexpr int kPair = 2;
constexpr int kUnit = 16 * kPair;

template <int M_, int G_, int S_>
struct SubCfg {
  static constexpr int M = M_;  // tokens per tile
  static constexpr int G = G_;  // trees per workgroup
  static constexpr int S = S_;  // subtrees per tree (2^k)
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRowBytes = 64;             // one K step of a bf16 row
  static constexpr int R = G * S * 16;             // subtree rows per stage
  static constexpr int kXBytes = M * kRowBytes;    // x rows of one stage
  static constexpr int kWBytes = R * kRowBytes;    // node rows of one stage
  static constexpr int kSlots = M + kUnit * S;     // group slots per tree (bound)
  static constexpr int kMaxGroups = G * (M / 16 + kPair * S);
  static constexpr int kMaxUnits = kMaxGroups / kPair;
  static constexpr int kMaxG = kPair * ((kMaxUnits + kWaves - 1) / kWaves);  // per wave
  static constexpr int kXLoads = M / 16 / kWaves;  // wave-wide loads per stage
  static constexpr int kWLoads = R / 16 / kWaves;
  static constexpr int kKeys = S * kClasses;       // (subtree, token class) keys
  static constexpr int kChunks = M / kWave;        // 64-token chunks of the tile
  static_assert(M % (16 * kWaves) == 0 && R % (16 * kWaves) == 0, "loads split over waves");
  static_assert(M <= kThreads && M % kWave == 0, "one thread per token while grouping");
  static_assert(G * S == 32, "one lane per (tree, subtree) item while listing groups");
  // LDS carve-up (bytes).
  static constexpr size_t kOffX = 0;                                    // 2 stages of x
  static constexpr size_t kOffW = kOffX + 2 * size_t(kXBytes);          // 2 stages of rows
  static constexpr size_t kOffPerm = kOffW + 2 * size_t(kWBytes);       // int16 [G][kSlots]
  static constexpr size_t kOffGroups = kOffPerm + size_t(G) * kSlots * 2;  // int32 [kMaxGroups]
  static constexpr size_t kOffBias = kOffGroups + size_t(kMaxGroups) * 4;  // f32 [G][S][16]
  static constexpr size_t kOffWcnt = kOffBias + size_t(G) * S * 16 * 4;  // int32 [G][kChunks][kKeys]
  static constexpr size_t kOffCnt = kOffWcnt + size_t(G) * kChunks * kKeys * 4;  // int32 [G][kKeys]
  static constexpr size_t kOffBase = kOffCnt + size_t(G) * kKeys * 4;     // int32 [G][S]
  static constexpr size_t kOffMisc = kOffBase + size_t(G) * S * 4;        // int32 [4]
  static constexpr size_t kLds = kOffMisc + 16;
  static_assert(kLds <= 160 * 1024, "LDS");
  // The epilogue reuses the stage buffers: per wave 4 groups of 16 x 16 fp32.
  static_assert(size_t(kWaves) * 4 * 16 * 17 * 4 <= 2 * size_t(kXBytes) + 2 * size_t(kWBytes),
                "epilogue scratch");
};

// Heap id of local node j of the subtree rooted at global node r.
__device__ __forceinline__ int64_t sub_global(int64_t r, int j) {
  const int lvl = 31 - __clz(j + 1);  // floor(log2(j+1))
  return ((r + 1) << lvl) - 1 + (j - ((1 << lvl) - 1));
}

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (uint64_t(1) << lane) - 1; }

// Lanes of this wavefront whose valid token has the same key (self
// included): one ballot per key bit, kept where the lane's own bit agrees.
__device__ __forceinline__ uint64_t peers_with_key(bool valid, int key, int bits) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const bool on = (key >> b) & 1;
    const uint64_t m = __ballot(valid && on);
    peers &= on ? m : ~m;
  }
  return valid ? peers : 0;
}

// LDS written by some lanes of a wavefront, then read by others of the same
// wavefront: the wave's LDS operations complete in order once issued, so a
// wait for them and a compiler barrier suffice.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
}

// Group entry: tree (within the workgroup), subtree, first slot.
__device__ __forceinline__ int group_pack(int tl, int s, int slot) {
  return (tl << 24) | (s << 16) | slot;
}

template <class C, int SL>
__global__ __launch_bounds__(C::kThreads, 1) void subtree_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, const uint16_t* __restrict__ b,
    float* __restrict__ rec_logit, int32_t* __restrict__ rec_next,
    const uint8_t* __restrict__ alive, const float* __restrict__ part, int ncols, int T, int d,
    int P, int D, int k, int64_t N, int tree_groups) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int M = C::M, G = C::G, S = C::S;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  // Workgroups an XCD runs together (hardware sends block b to XCD b % 8)
  // share token tiles and tree groups: logical tile-major order.
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  const int tile = logical / tree_groups;
  const int p0 = (logical - tile * tree_groups) * G;
  const int t0 = tile * M;
  const int64_t first_sub = (int64_t(1) << k) - 1;  // heap id of subtree 0's root
  constexpr int kUsed = (1 << SL) - 1;              // subtree nodes

  int16_t* perm = reinterpret_cast<int16_t*>(lds + C::kOffPerm);
  int32_t* groups = reinterpret_cast<int32_t*>(lds + C::kOffGroups);
  float* bias = reinterpret_cast<float*>(lds + C::kOffBias);
  int32_t* wcnt = reinterpret_cast<int32_t*>(lds + C::kOffWcnt);
  int32_t* cnt = reinterpret_cast<int32_t*>(lds + C::kOffCnt);
  int32_t* sbase = reinterpret_cast<int32_t*>(lds + C::kOffBase);
  int32_t* misc = reinterpret_cast<int32_t*>(lds + C::kOffMisc);

  // Row starts of the direct-to-LDS loads (fixed over K): x rows clamped to
  // T-1, node rows of trees past P clamped to tree P-1, spare subtree
  // columns reading the subtree root's row (their results are unused).
  auto x_row = [&](int r) {
    const int t = t0 + r < T ? t0 + r : T - 1;
    return x + static_cast<int64_t>(t) * d;
  };
  auto w_row = [&](int r) {
    const int tl = r / (S * 16);
    const int s = (r / 16) % S;
    const int jj = (r & 15) < kUsed ? (r & 15) : 0;
    const int p = p0 + tl < P ? p0 + tl : P - 1;
    return W + (static_cast<int64_t>(p) * N + sub_global(first_sub + s, jj)) * d;
  };
  const int nk = d / 32;
  // Stage 0's loads do not depend on the grouping: issued first, so that
  // they are in flight together with the grouping's own reads.
  direct_load_rows_s<C, M, kSwz>(lds, C::kOffX, x_row, 0, wave, lane);
  direct_load_rows_s<C, C::R, kSwz>(lds, C::kOffW, w_row, 0, wave, lane);

  // ---- grouping: per tree, the tile's tokens by level-k node ----
  // One thread per token of the tile (M <= threads).  For every tree of the
  // group at once: the token's subtree s and row residue form the key
  // s * 16 + residue; equal keys within a wavefront find each other by
  // ballots, and per-wavefront counts go to LDS.
  constexpr int kKeyBits = __builtin_ctz(S) + __builtin_ctz(kClasses);
  const int t = t0 + tid;
  const bool tok_ok = tid < M && t < T;
  int sub[G];
  if (part) {
    // Levels 0..k-1 from the dense product's two K halves (column p*S + n
    // of tree p's node n, token-fastest: part[(half*ncols + col)*T + t]):
    // logits summed, bias added and walked here, as the dense product's own
    // epilogue does otherwise; their records written beside levels k..D.
    float tb[G][S];  // top nodes' biases (the same for every token)
#pragma unroll
    for (int tl = 0; tl < G; ++tl)
#pragma unroll
      for (int n = 0; n < S; ++n) {
        const int p = p0 + tl < P ? p0 + tl : P - 1;
        tb[tl][n] = n < S - 1 ? bf16_to_f32(b[static_cast<int64_t>(p) * N + n]) : 0.0f;
      }
    float lg[G][S];
    const int tt = tok_ok ? t : 0;
#pragma unroll
    for (int tl = 0; tl < G; ++tl)
#pragma unroll
      for (int n = 0; n < S; ++n) {
        const int p = p0 + tl < P ? p0 + tl : P - 1;
        const int64_t c = static_cast<int64_t>(p) * S + n;
        lg[tl][n] = part[c * T + tt] + part[(ncols + c) * T + tt];
      }
#pragma unroll
    for (int tl = 0; tl < G; ++tl) {
      sub[tl] = -1;
      if (tok_ok && p0 + tl < P) {
        float* out = rec_logit + (static_cast<int64_t>(p0 + tl) * T + t) * (D + 1);
        int n = 0;
#pragma unroll
        for (int lv = 0; lv < __builtin_ctz(S); ++lv) {  // S = 2^k
          float a = 0.0f;
#pragma unroll
          for (int j = 0; j < S - 1; ++j)
            if (j == n) a = lg[tl][j] + tb[tl][j];
          out[lv] = a;
          n = 2 * n + 1 + go_right(a);
        }
        sub[tl] = n - static_cast<int>(first_sub);
      }
    }
  } else {
#pragma unroll
    for (int tl = 0; tl < G; ++tl)
      sub[tl] = tok_ok && p0 + tl < P
                    ? rec_next[static_cast<int64_t>(p0 + tl) * T + t] - static_cast<int>(first_sub)
                    : -1;
  }
  for (int i = tid; i < G * C::kSlots; i += C::kThreads) perm[i] = -1;
  for (int i = tid; i < G * C::kChunks * C::kKeys; i += C::kThreads) wcnt[i] = 0;
  for (int i = tid; i < G * S * 16; i += C::kThreads) {
    const int tl = i / (S * 16);
    const int s = (i / 16) % S;
    const int j = i & 15;
    const int p = p0 + tl;
    float v = 0.0f;
    if (p < P && j < kUsed) v = bf16_to_f32(b[static_cast<int64_t>(p) * N + sub_global(first_sub + s, j)]);
    bias[i] = v;
  }
  __syncthreads();
  const int res = tid & (kClasses - 1);
  const int chunk = tid / kWave;
  int rank[G];
#pragma unroll
  for (int tl = 0; tl < G; ++tl) {
    const bool valid = sub[tl] >= 0;
    const int key = (valid ? sub[tl] : 0) * kClasses + res;
    const uint64_t peers = peers_with_key(valid, key, kKeyBits);
    rank[tl] = __popcll(peers & lanes_below(lane));
    if (valid && rank[tl] == 0)
      wcnt[(tl * C::kChunks + chunk) * C::kKeys + key] = __popcll(peers);
  }
  __syncthreads();
  // Per (tree, key): exclusive prefix over the 64-token chunks, and the total.
  for (int i = tid; i < G * C::kKeys; i += C::kThreads) {
    const int tl = i / C::kKeys;
    const int kk = i - tl * C::kKeys;
    int run = 0;
    for (int c = 0; c < C::kChunks; ++c) {
      int32_t* w = wcnt + (tl * C::kChunks + c) * C::kKeys + kk;
      const int v = *w;
      *w = run;
      run += v;
    }
    cnt[i] = run;
  }
  __syncthreads();
  // Groups: lane i of wave 0 takes item i = (tree i / S, subtree i % S); its
  // token count padded to whole units; a scan within the tree gives the
  // subtree's first slot, a scan over all items its first group.
  if (tid < 32) {
    const int tl = tid / S;
    const int s = tid % S;
    int n = 0;
#pragma unroll
    for (int r = 0; r < kClasses; ++r) n += cnt[tl * C::kKeys + s * kClasses + r];
    const int pad = (n + kUnit - 1) & ~(kUnit - 1);
    int slot = pad, gi = pad / 16;  // inclusive scans
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const int o_slot = __shfl_up(slot, off, 32);
      const int o_gi = __shfl_up(gi, off, 32);
      if (s >= off) slot += o_slot;
      if (tid >= off) gi += o_gi;
    }
    slot -= pad;
    gi -= pad / 16;
    sbase[tid] = slot;
    for (int g = 0; g < pad / 16; ++g) groups[gi + g] = group_pack(tl, s, slot + 16 * g);
    if (tid == 31) misc[0] = gi + pad / 16;
  }
  __syncthreads();
  // Each token's slot: order within its subtree by (rank within the class,
  // class), so that consecutive slots take distinct classes while the
  // counts allow.
#pragma unroll
  for (int tl = 0; tl < G; ++tl) {
    if (sub[tl] >= 0) {
      const int key = sub[tl] * kClasses + res;
      const int r = wcnt[(tl * C::kChunks + chunk) * C::kKeys + key] + rank[tl];
      const int32_t* cs = cnt + tl * C::kKeys + sub[tl] * kClasses;
      int pos = sbase[tl * S + sub[tl]];
#pragma unroll
      for (int qq = 0; qq < kClasses; ++qq) {
        const int c = cs[qq];
        pos += c < r ? c : r;
        pos += (qq < res && c > r) ? 1 : 0;
      }
      perm[tl * C::kSlots + pos] = static_cast<int16_t>(tid);
    }
  }
  __syncthreads();

  // ---- this wave's groups: operand addresses ----
  // Slots past the wave's count read valid rows and their products are
  // dropped, so the K loop has no branch.
  // Whole units per wave (a unit's groups share their subtree rows).
  const int nu_all = misc[0] / kPair;
  const int ubeg = (wave * nu_all) / C::kWaves;
  const int gbeg = kPair * ubeg;
  const int ng = kPair * (((wave + 1) * nu_all) / C::kWaves - ubeg);
  const int m = lane & 15;
  const int q = lane >> 4;
  uint32_t addrA[C::kMaxG], addrB[C::kMaxG];
#pragma unroll
  for (int g = 0; g < C::kMaxG; ++g) {
    const int e = g < ng ? groups[gbeg + g] : 0;
    const int tl = e >> 24;
    const int s = (e >> 16) & 0xff;
    const int slot = e & 0xffff;
    int row = perm[tl * C::kSlots + slot + m];
    row = row < 0 ? 0 : row;
    addrA[g] = static_cast<uint32_t>(row * C::kRowBytes + ((q ^ lds_swz_s<kSwz>(row)) << 4));
    const int brow = (tl * S + s) * 16 + m;
    addrB[g] = static_cast<uint32_t>(brow * C::kRowBytes + ((q ^ lds_swz_s<kSwz>(brow)) << 4));
  }
  f32x4_t acc[C::kMaxG];
#pragma unroll
  for (int g = 0; g < C::kMaxG; ++g) acc[g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- main loop: two stages, one barrier per K step ----
  // Iteration ks issues the loads of stage ks+1 into buffer (ks+1) % 2, then
  // works on stage ks (stage 0 was issued before the grouping).  Each
  // wave-wide load fills 16 rows of 64 bytes, chunks XOR-swizzled by row
  // bits 1-2.
  for (int ks = 0; ks < nk; ++ks) {
    wait_vmcnt<0>();   // this wave's loads of stage ks have landed
    stage_barrier();   // everyone's have; everyone is done with stage ks-1
    if (ks + 1 < nk) {
      const int buf = (ks + 1) & 1;
      direct_load_rows_s<C, M, kSwz>(lds, C::kOffX + buf * C::kXBytes, x_row, (ks + 1) * 32, wave,
                                     lane);
      direct_load_rows_s<C, C::R, kSwz>(lds, C::kOffW + buf * C::kWBytes, w_row, (ks + 1) * 32,
                                        wave, lane);
    }
    const unsigned char* xs = lds + C::kOffX + (ks & 1) * C::kXBytes;
    const unsigned char* ws = lds + C::kOffW + (ks & 1) * C::kWBytes;
#pragma unroll
    for (int u = 0; u < C::kMaxG; u += kPair) {
      const bf16x8_t bfrag = *reinterpret_cast<const bf16x8_t*>(ws + addrB[u]);
#pragma unroll
      for (int g = u; g < u + kPair; ++g) {
        const bf16x8_t afrag = *reinterpret_cast<const bf16x8_t*>(xs + addrA[g]);
        // D[token][node]: lane l holds tokens 4(l/16)+i of node l%16.
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag, acc[g], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // stage buffers free for the epilogue

  // ---- epilogue: 4 groups at a time per wave through LDS ----
  constexpr int kPitch = 17;  // floats per staged token row (16 nodes + pad)
  float* ep = reinterpret_cast<float*>(lds) + wave * 4 * 16 * kPitch;
  const int L = D + 1;
#pragma unroll
  for (int g4 = 0; g4 < C::kMaxG; g4 += 4) {
    if (g4 < ng) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (g4 + u < C::kMaxG && g4 + u < ng) {
#pragma unroll
          for (int i = 0; i < 4; ++i) ep[(u * 16 + 4 * q + i) * kPitch + m] = acc[g4 + u][i];
        }
      }
      wave_lds_sync();
      const int u = lane >> 4;  // group of this lane's token
      const int g = g4 + u;
      if (g < ng) {
        const int e = groups[gbeg + g];
        const int tl = e >> 24;
        const int s = (e >> 16) & 0xff;
        const int slot = e & 0xffff;
        const int row = perm[tl * C::kSlots + slot + m];
        if (row >= 0) {
          const int p = p0 + tl;
          const int t = t0 + row;
          const float* lg = ep + (u * 16 + m) * kPitch;
          const float* bs = bias + (tl * S + s) * 16;
          const int64_t root = first_sub + s;
          float out[4];
          int j = 0;
#pragma unroll
          for (int lv = 0; lv < SL; ++lv) {
            const float a = lg[j] + bs[j];
            out[lv] = a;
            if (lv + 1 < SL) {
              int rr = go_right(a);
              if (alive && !alive[static_cast<int64_t>(p) * N + sub_global(root, 2 * j + 1 + rr)])
                rr ^= 1;  // pruned child: its sibling
              j = 2 * j + 1 + rr;
            }
          }
          float* dst = rec_logit + (static_cast<int64_t>(p) * T + t) * L + k;
#pragma unroll
          for (int lv = 0; lv < SL; ++lv) dst[lv] = out[lv];
          rec_next[static_cast<int64_t>(p) * T + t] = static_cast<int32_t>(sub_global(root, j));
        }
      }
      wave_lds_sync();  // reads done before the next four groups are staged
    }
  }
}

template <int M, int G, int S>
using Cfg = SubCfg<M, G, S>;

// Tile shape per subtree count: G * S * 16 = 512 node rows per stage, and at
// most about 20 groups (accumulator blocks) per wave.
template <int S> struct SubPick;
template <> struct SubPick<2> { using C = Cfg<128, 16, 2>; };
template <> struct SubPick<4> { using C = Cfg<256, 8, 4>; };
template <> struct SubPick<8> { using C = Cfg<512, 4, 8>; };
template <> struct SubPick<16> { using C = Cfg<512, 2, 16>; };
template <> struct SubPick<32> { using C = Cfg<512, 1, 32>; };

template <int S, int SL>
hipError_t launch_sub(const Dims& s, int k, const void* x, const void* W, const void* b,
                      float* rec_logit, int32_t* rec_next, const float* part, int ncols,
                      hipStream_t st) {
  using C = typename SubPick<S>::C;
  auto kern = subtree_kernel<C, SL>;
  {
    const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), int(C::kLds));
    if (e != hipSuccess) return e;
  }
  const int tiles = static_cast<int>((s.T + C::M - 1) / C::M);
  const int tree_groups = (s.P + C::G - 1) / C::G;
  const int64_t blocks = int64_t(tiles) * tree_groups;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  kern<<<dim3(static_cast<unsigned>(blocks)), dim3(C::kThreads), C::kLds, st>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W),
      static_cast<const uint16_t*>(b), rec_logit, rec_next, s.prune ? s.prune->alive : nullptr,
      part, ncols, static_cast<int>(s.T), s.d, s.P, s.D, k, s.N, tree_groups);
  return hipGetLastError();
}

template <int S>
hipError_t launch_sub_s(const Dims& s, int k, const void* x, const void* W, const void* b,
                        float* rec_logit, int32_t* rec_next, const float* part, int ncols,
                        hipStream_t st) {
  switch (s.D - k + 1) {
    case 1: return launch_sub<S, 1>(s, k, x, W, b, rec_logit, rec_next, part, ncols, st);
    case 2: return launch_sub<S, 2>(s, k, x, W, b, rec_logit, rec_next, part, ncols, st);
    case 3: return launch_sub<S, 3>(s, k, x, W, b, rec_logit, rec_next, part, ncols, st);
    case 4: return launch_sub<S, 4>(s, k, x, W, b, rec_logit, rec_next, part, ncols, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool subtree_supported(const Dims& s, int k) {
  // 32-wide K steps; 1..4 subtree levels; 2..32 subtrees per tree; 16-bit
  // group slots; element offsets of x within 63 bits (always).
  return s.dtype == 1 && s.d % 32 == 0 && k >= 1 && k <= 5 && k <= s.D && s.D - k + 1 <= 4 &&
         s.T >= 1;
}

hipError_t launch_subtree(const Dims& s, int k, const void* x, const void* W, const void* b,
                          float* rec_logit, int32_t* rec_next, const float* part, int ncols,
                          hipStream_t st) {
  switch (k) {
    case 1: return launch_sub_s<2>(s, k, x, W, b, rec_logit, rec_next, part, ncols, st);
    case 2: return launch_sub_s<4>(s, k, x, W, b, rec_logit, rec_next, part, ncols, st);
    case 3: return launch_sub_s<8>(s, k, x, W, b, rec_logit, rec_next, part, ncols, st);
    case 4: return launch_sub_s<16>(s, k, x, W, b, rec_logit, rec_next, part, ncols, st);
    case 5: return launch_sub_s<32>(s, k, x, W, b, rec_logit, rec_next, part, ncols, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fff
