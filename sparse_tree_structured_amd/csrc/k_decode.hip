// Decode-shaped FFF forward (T <= 64 tokens) on gfx950: the whole layer in
// one launch.
//
// At decode sizes the layer is bound by reading W_out (P*h x d) and by the
// chain of dependent node evaluations down each tree (explainer page,
// section 2: one root-to-leaf path per tree, the sign of each visited node's
// logit choosing the child).  The launch holds two kinds of workgroups,
// routing ones first (lower block ids), and overlaps the two:
//
//  routing     item = (tree p, up to 16 tokens).  The walk proceeds in
//              rounds.  A round evaluates, below every distinct node the
//              item's tokens sit on, the subtree of the next rl levels (rl
//              chosen so that at most 16 node rows are read), as one
//              16-row x 16-token product on the matrix cores with the model
//              width split over the four waves (each wave keeps its slice of
//              the token rows in registers for all rounds).  The round's V
//              rows and biases arrive in the same round trip.  Wave 0 sums
//              the four partial logits, walks the tokens through the subtree
//              (a < 0 goes left) and plans the next round; the GELU(a) * v_n
//              terms of the visited nodes (GELU before the sum: section 3.C)
//              are added to the token's H row while the next round's loads
//              are in flight.  H[t, p*h:(p+1)*h] (workspace, bf16 as in the
//              prefill path) and path_out are written, then the item is
//              published.
//  projection  item = (K chunk of 512 rows, 64 output columns).  The
//              workgroup streams its W_out block into LDS transposed
//              ([n][k]), waits until the routing items of the trees in its K
//              chunk are published, forms the partial y block H[:, chunk] .
//              block on the matrix cores and writes it to the workspace; the
//              last partial of a column slice to arrive sums them in chunk
//              order and writes y in bf16.
//
// Workgroups hand data to each other through the workspace with device-
// coherent (sc1) 16-byte buffer loads and stores, which do not stay in one
// XCD's L2, so no L2 write-back or invalidation is needed: a writer waits
// until its stores have completed, then publishes by storing the call's
// epoch into a slot of its own (routing items; split-K partials).  A slot
// that does not hold the current epoch counts as not done, so nothing needs
// clearing between calls or before the first one.
//
// Epochs.  An ordinary call gets a fresh one from the host (a per-process
// counter started at a random point) and records it in the workspace
// header.  A call captured into a graph cannot take a new value from the
// host on each replay, so it reads the header at entry instead and uses the
// next value; the workgroup that sees every partial of the call arrived
// (which implies every workgroup has read the header) stores the call's
// epoch back.  A header that fails its check word (a fresh workspace) gives
// the launch's own value.
//
// A projection workgroup only waits on routing workgroups, which have lower
// block ids, never wait themselves and are all resident (the grid is capped
// at what the device holds at once); the wait is also bounded.  A wait that
// gives up poisons the workgroup's partial with NaN (so the columns of y it
// feeds come out NaN) and marks its arrival slot.  In a captured call that
// mark turns the header into a poisoned state: a routing workgroup that
// starts only after the call was finished off would otherwise read the
// advanced header and publish with the next replay's epoch; in the poisoned
// state every workgroup only writes NaN to y, until an ordinary call
// rewrites the header.
#include <atomic>
#include <chrono>
#include <random>

#include "common.hpp"
#include "fff.h"
#include "launch.hpp"
#include "mfma_tile.hpp"

namespace fff {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kDecTok = 16;       // most tokens per routing item (one MFMA column block)
constexpr int kKc = 512;          // projection: K rows per item
constexpr int kColSlice = 64;     // projection: output columns per item
constexpr int kMaxRows = 16;      // node rows per routing round (one MFMA row block)
constexpr int kMaxLevels = 16;    // D + 1
constexpr int kMaxD = 2048;       // model width: 16 k-steps per wave slice
constexpr int kMaxH = 256;        // node output width: 2 H pieces per thread
constexpr int kHPieces = kDecTok * (kMaxH / 8) / kDecThreads;
constexpr int kWtPitch = kKc + 8;
// Epochs are 62-bit and never 0.  Those of ordinary calls have bit 61 set
// (random values), those a captured call derives from the header have it
// clear, so the two kinds never meet.
constexpr uint64_t kEpochMask = (uint64_t(1) << 62) - 1;
constexpr uint64_t kDeviceEpochMask = (uint64_t(1) << 61) - 1;
constexpr uint64_t kHostEpochBit = uint64_t(1) << 61;
constexpr uint64_t kGaveUp = uint64_t(1) << 63;  // arrival slot: the partial's wait gave up
// Header check words: header[1] = header[0] ^ one of these.
constexpr uint64_t kHdrValid = 0x6A09E667F3BCC908ull;
constexpr uint64_t kHdrPoison = 0xBB67AE8584CAA73Bull;
constexpr int kSpinLimit = 1 << 22;
constexpr int kTestSpinLimit = 64;
constexpr int kSc1 = 16;  // buffer cache policy: device scope (sc1)

struct DecodeArgs {
  const uint16_t* x;
  const uint16_t* W;
  const uint16_t* b;
  const uint16_t* V;
  const uint16_t* Wout;
  uint16_t* y;
  int32_t* path_out;
  uint16_t* H;       // workspace [T, K] bf16
  float* partial;    // workspace [K / kKc, T, d] fp32
  uint64_t* done;    // workspace [routing items] epoch of the call that routed it
  uint64_t* arrive;  // workspace [d / kColSlice][K / kKc] epoch of the call whose partial
                     // arrived, | kGaveUp if its wait gave up
  uint64_t* hdr;     // workspace header: [0] epoch of the last call, [1] check word
  uint64_t seed;     // the call's epoch (ordinary call), or the one to use when the header
                     // fails its check (captured call)
  int device_epoch;  // 1: captured call, epoch from the header
  int publish;       // 0: routing items are not published (give-up test)
  int spin_limit;    // polls of a projection wait
  int T, d, P, D, h, K;
  int64_t N;
  int n_route_wg, n_proj_wg;
  int tok;               // tokens per routing item (<= kDecTok)
  int post;              // 1: GELU on the summed h-vector instead of on each node's logit
  const uint8_t* alive;  // static pruning: [P][N] 1 = node alive; null = every node
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ uint32_t word(const uint4& q, int i) {
  return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// Heap id of local node j (heap order within the subtree) of the subtree
// rooted at global node r.
__device__ __forceinline__ int64_t sub_global(int64_t r, int j) {
  const int lvl = 31 - __clz(j + 1);
  return ((r + 1) << lvl) - 1 + (j - ((1 << lvl) - 1));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// Plain buffer loads.  A lane whose offset is kOob (past every buffer's
// size) gets zeros, so loads need no per-lane branch: branches around loads
// make the compiler wait for all outstanding loads where they join.
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint16_t buffer_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint8_t buffer_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ uint4 coherent_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}
__device__ __forceinline__ void coherent_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kSc1);
}

// One wave waits (at most `limit` polls) until slots [first, first + n) all
// hold `epoch`; false if it gave up.
__device__ bool wait_slots(const uint64_t* done, int first, int n, uint64_t epoch, int limit) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int it = 0; it < limit; ++it) {
    bool ok = true;
    for (int i = lane; i < n; i += kWave)
      ok &= __hip_atomic_load(done + first + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
    if (__all(ok)) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// LDS: the two roles overlay one allocation.
struct ProjLds {
  static constexpr size_t wt = 0;  // [64][kWtPitch] bf16
  static constexpr size_t total = size_t(kColSlice) * kWtPitch * 2;
};
struct RouteLds {
  static constexpr size_t part = 0;                                 // [3 waves][16][16] f32
  static constexpr size_t lgs = part + 3 * 256 * 4;                 // [16 rows][16 tok] f32 logit
  static constexpr size_t vc = lgs + 256 * 4;                       // [2][16 rows][h] bf16
  static constexpr size_t rows = vc + 2 * size_t(kMaxRows) * kMaxH * 2;  // [16] i32 node ids
  static constexpr size_t roots = rows + kMaxRows * 4;              // [16] i32
  static constexpr size_t rsm = roots + kDecTok * 4;                // [16 tok][4] i32 row
  static constexpr size_t meta = rsm + kDecTok * 4 * 4;             // R, rl
  static constexpr size_t total = meta + 16;
};
constexpr size_t kDecLds = ProjLds::total > RouteLds::total ? ProjLds::total : RouteLds::total;

// Adds one round's GELU(a) * v_n terms (a * v_n when `post`) to the thread's
// H pieces (token m, eight columns c0..c0+7; piece i is thread + 256 i).  rsm
// holds the rows token m visited this round, lgs the round's logits
// [row][token].
__device__ __forceinline__ void add_h_terms(const unsigned char* lds, const uint16_t* vcb, int rl,
                                            int nt, int h, int post,
                                            float (&hacc)[kHPieces][8]) {
  const float* lgs = reinterpret_cast<const float*>(lds + RouteLds::lgs);
  const int32_t* rsm = reinterpret_cast<const int32_t*>(lds + RouteLds::rsm);
  const int hc = h / 8;
#pragma unroll
  for (int i = 0; i < kHPieces; ++i) {
    const int e = threadIdx.x + i * kDecThreads;
    const int m = e / hc;
    if (m < nt) {
      const int c0 = (e - m * hc) * 8;
      for (int lv = 0; lv < rl; ++lv) {
        const int row = rsm[m * 4 + lv];
        const float lg = lgs[row * 16 + m];
        const float g = post ? lg : gelu_tanh(lg);
        const uint4 v = *reinterpret_cast<const uint4*>(vcb + row * h + c0);
        hacc[i][0] += g * bf16lo(v.x);
        hacc[i][1] += g * bf16hi(v.x);
        hacc[i][2] += g * bf16lo(v.y);
        hacc[i][3] += g * bf16hi(v.y);
        hacc[i][4] += g * bf16lo(v.z);
        hacc[i][5] += g * bf16hi(v.z);
        hacc[i][6] += g * bf16lo(v.w);
        hacc[i][7] += g * bf16hi(v.w);
      }
    }
  }
}

// Routing of one item: tree p, tokens [t0, t0 + nt), published with epoch e.
__device__ void route_item(const DecodeArgs& a, unsigned char* lds, int item, int p, int t0,
                           int nt, uint64_t e) {
  float* part = reinterpret_cast<float*>(lds + RouteLds::part);
  float* lgs = reinterpret_cast<float*>(lds + RouteLds::lgs);
  uint16_t* vc = reinterpret_cast<uint16_t*>(lds + RouteLds::vc);
  int32_t* rows = reinterpret_cast<int32_t*>(lds + RouteLds::rows);
  int32_t* roots = reinterpret_cast<int32_t*>(lds + RouteLds::roots);
  int32_t* rsm = reinterpret_cast<int32_t*>(lds + RouteLds::rsm);
  int32_t* meta = reinterpret_cast<int32_t*>(lds + RouteLds::meta);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int j = lane & 15;  // node row of the block (A) / token (B)
  const int q = lane >> 4;  // 8-wide k group within each 32-wide step
  const int klen = a.d / kDecWaves;
  const int nsteps = klen / 32;  // <= 16
  const int hc = a.h / 8;
  const int vc_stride = kMaxRows * a.h;
  const __amdgpu_buffer_rsrc_t xbuf = buffer_of(a.x, uint32_t(a.T) * a.d * 2);
  const __amdgpu_buffer_rsrc_t wbuf =
      buffer_of(a.W + static_cast<int64_t>(p) * a.N * a.d, uint32_t(a.N) * a.d * 2);
  const __amdgpu_buffer_rsrc_t bbuf = buffer_of(a.b + static_cast<int64_t>(p) * a.N, uint32_t(a.N) * 2);
  const __amdgpu_buffer_rsrc_t vbuf =
      buffer_of(a.V + static_cast<int64_t>(p) * a.N * a.h, uint32_t(a.N) * a.h * 2);
  // Node alive flags of this tree (an empty buffer when nothing is pruned:
  // its loads return 0 and are then read as alive).
  const __amdgpu_buffer_rsrc_t abuf =
      buffer_of(a.alive ? static_cast<const void*>(a.alive + static_cast<int64_t>(p) * a.N)
                        : static_cast<const void*>(a.x),
                a.alive ? uint32_t(a.N) : 0);

  // Byte offset of this lane's slice of its token row (rows past nt repeat
  // the last token; their results are not used; k steps past the width load
  // zeros).
  const uint32_t xoff = uint32_t((t0 + (j < nt ? j : nt - 1)) * a.d + wave * klen + q * 8) * 2;
  uint4 xf[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) xf[u] = buffer_load16(xbuf, u < nsteps ? xoff + u * 64 : kOob);
  float hacc[kHPieces][8];
#pragma unroll
  for (int i = 0; i < kHPieces; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) hacc[i][c] = 0.0f;

  // Round 1 evaluates the top subtree, the same for every token: its rows
  // are heap ids 0 .. S-1.  Wave 0 keeps, in lane j, token j's current node,
  // the index of its subtree root in this round, and its last visited node.
  int rl = a.D + 1 < 4 ? a.D + 1 : 4;
  int R = (1 << rl) - 1;
  int cur = 0, troot = 0, last_node = 0;
  int prev_rl = 0, buf = 0;
  // The first round's rows are heap ids 0 .. S-1 (every earlier reader of
  // rows[] passed the previous item's last barrier).
  if (tid < kMaxRows) rows[tid] = tid;
  __syncthreads();  // LDS of a previous item is no longer read

  for (int lev = 0;;) {
    const int S = (1 << rl) - 1;
    // Node ids of the rows this lane reads (LDS reads issued together, then
    // one wait): its W row and alive flags (row j; rows past R repeat row
    // 0, unused), its V pieces, and the biases of rows 4q .. 4q+3 (wave 0).
    const int rw = j < R ? j : 0;
    const int node_w = rows[rw];
    int rv[kHPieces], node_v[kHPieces];
#pragma unroll
    for (int i = 0; i < kHPieces; ++i) {
      const int e = tid + i * kDecThreads;
      rv[i] = e / hc < R ? e / hc : R - 1;
      node_v[i] = rows[rv[i]];
    }
    int node_b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) node_b[r] = rows[4 * q + r < R ? 4 * q + r : 0];
    uint4 wf[16];
    {
      const uint32_t woff = uint32_t(node_w * a.d + wave * klen + q * 8) * 2;
#pragma unroll
      for (int u = 0; u < 16; ++u) wf[u] = buffer_load16(wbuf, u < nsteps ? woff + u * 64 : kOob);
    }
    uint4 vr[kHPieces];
#pragma unroll
    for (int i = 0; i < kHPieces; ++i) {
      const int e = tid + i * kDecThreads;
      vr[i] = buffer_load16(
          vbuf, e < R * hc ? uint32_t(node_v[i] * a.h + (e - rv[i] * hc) * 8) * 2 : kOob);
    }
    // Raw bias bits of rows 4q .. 4q+3 (used by wave 0), converted only
    // after the MFMA so that nothing waits on these loads before then.
    uint16_t braw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      braw[r] = buffer_load2(bbuf, 4 * q + r < R ? uint32_t(node_b[r]) * 2 : kOob);
    // Alive flags of both children of row j (wave 0, lanes j < R; rows at
    // the leaf level read past the buffer and get 0, never used).
    uint8_t child_l, child_r;
    {
      const uint32_t off =
          wave == 0 && q == 0 && j < R ? uint32_t(2 * node_w + 1) : kOob;
      child_l = buffer_load1(abuf, off);
      child_r = buffer_load1(abuf, off == kOob ? kOob : off + 1);
    }
    // The previous round's H terms, while these loads are in flight.
    if (prev_rl) add_h_terms(lds, vc + (buf ^ 1) * vc_stride, prev_rl, nt, a.h, a.post, hacc);

    // k steps past the width have zero operands.
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 16; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wf[u]), as_bf16x8(xf[u]), acc, 0, 0, 0);
    // acc[r] = this wave's partial logit of row 4q + r for token j.
    if (wave != 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) part[((wave - 1) * 16 + 4 * q + r) * 16 + j] = acc[r];
    }
#pragma unroll
    for (int i = 0; i < kHPieces; ++i) {
      const int e = tid + i * kDecThreads;
      if (e < R * hc) {
        const int r = e / hc;
        *reinterpret_cast<uint4*>(vc + buf * vc_stride + r * a.h + (e - r * hc) * 8) = vr[i];
      }
    }
    __syncthreads();

    if (wave == 0) {
      // Logits (partials summed in wave order); the sign of row 4q + r for
      // token j becomes bit 16q + j of ballot r.
      uint64_t right[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        const float lg = acc[r] + part[(0 * 16 + row) * 16 + j] + part[(1 * 16 + row) * 16 + j] +
                         part[(2 * 16 + row) * 16 + j] + bf16_to_f32(braw[r]);
        lgs[row * 16 + j] = lg;
        right[r] = __ballot(go_right(lg));
      }
      // Bit r of alive_l / alive_r: the left / right child of row r is alive.
      const uint64_t alive_l = __ballot(lane < 16 && (!a.alive || child_l != 0));
      const uint64_t alive_r = __ballot(lane < 16 && (!a.alive || child_r != 0));
      // Walk of token j through its subtree (the four lanes of token j do
      // the same walk; lane q == 0 records the visited rows).
      const int base = troot * S;
      int jj = 0, row = 0, bit = 0;
      for (int lv = 0; lv < rl; ++lv) {
        row = base + jj;
        const int sel = row & 3;
        const uint64_t m = sel == 0 ? right[0] : sel == 1 ? right[1] : sel == 2 ? right[2] : right[3];
        bit = static_cast<int>((m >> ((row >> 2) * 16 + j)) & 1);
        // Static pruning: a step into a pruned child goes to its sibling.
        if (!(((bit ? alive_r : alive_l) >> row) & 1)) bit ^= 1;
        if (q == 0 && j < nt) rsm[j * 4 + lv] = row;
        jj = 2 * jj + 1 + bit;
      }
      last_node = rows[row];
      cur = 2 * last_node + 1 + bit;
      if (lev + rl <= a.D) {
        // Plan of the next round: distinct current nodes of the tokens
        // (lanes 0..nt-1 hold tokens 0..nt-1), the depth of the subtrees
        // below them, and their rows (subtree of root i at rows
        // i*S' .. i*S'+S'-1).  Every lane of token j finds the same root.
        int f = -1;  // lowest token with the same node
#pragma unroll
        for (int k = 0; k < kDecTok; ++k) {
          const int ck = __builtin_amdgcn_readlane(cur, k);
          if (k < nt && f < 0 && ck == cur) f = k;
        }
        const uint64_t firsts = __ballot(lane < nt && f == lane);
        const int n = __popcll(firsts);
        const int rank = f < 0 ? 0 : __popcll(firsts & ((uint64_t(1) << f) - 1));
        if (lane < nt && f == lane) roots[rank] = cur;
        troot = j < nt ? rank : 0;
        int nrl = a.D + 1 - (lev + rl);
        nrl = nrl < 4 ? nrl : 4;
        while (nrl > 1 && n * ((1 << nrl) - 1) > kMaxRows) --nrl;
        const int nS = (1 << nrl) - 1;
        // LDS operations of one wave complete in order: roots[] is written.
        if (lane < n * nS) rows[lane] = static_cast<int32_t>(sub_global(roots[lane / nS], lane % nS));
        if (lane == 0) {
          meta[0] = n * nS;
          meta[1] = nrl;
        }
      }
    }
    // Every load of this round has been consumed (some only by some waves
    // or lanes): wait for all of them here, so that the compiler, which
    // cannot tell, does not make the loop head wait for outstanding loads;
    // on entry that would hold round 1's node rows behind the token rows.
    wait_vmcnt<0>();
    __syncthreads();
    lev += rl;
    prev_rl = rl;
    buf ^= 1;
    if (lev > a.D) break;
    R = meta[0];
    rl = meta[1];
  }
  add_h_terms(lds, vc + (buf ^ 1) * vc_stride, prev_rl, nt, a.h, a.post, hacc);

  const __amdgpu_buffer_rsrc_t hbuf = buffer_of(a.H, uint32_t(a.T) * a.K * 2);
#pragma unroll
  for (int i = 0; i < kHPieces; ++i) {
    const int e = tid + i * kDecThreads;
    const int m = e / hc;
    if (m < nt) {
      const int c0 = (e - m * hc) * 8;
      if (a.post) {
#pragma unroll
        for (int u = 0; u < 8; ++u) hacc[i][u] = gelu_tanh(hacc[i][u]);
      }
      coherent_store16(hbuf, uint32_t((t0 + m) * a.K + p * a.h + c0) * 2,
                       make_uint4(pack_bf16x2(hacc[i][0], hacc[i][1]),
                                  pack_bf16x2(hacc[i][2], hacc[i][3]),
                                  pack_bf16x2(hacc[i][4], hacc[i][5]),
                                  pack_bf16x2(hacc[i][6], hacc[i][7])));
    }
  }
  if (a.path_out && wave == 0 && q == 0 && j < nt)
    a.path_out[static_cast<int64_t>(t0 + j) * a.P + p] = last_node - ((1 << a.D) - 1);

  // Publish the item once every thread's stores have completed.
  wait_vmcnt<0>();
  __syncthreads();
  if (tid == 0 && a.publish)
    __hip_atomic_store(a.done + item, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// W_out block (K chunk kc, column slice cs) into LDS as wt[n][k].  A thread
// takes 4(k) x 8(n) pieces (four 16-byte row loads, byte permutes, eight
// 8-byte LDS writes); eight lanes cover one 128-byte row segment.
__device__ void load_wout_block(const DecodeArgs& a, unsigned char* lds, int kc, int cs) {
  uint16_t* wt = reinterpret_cast<uint16_t*>(lds + ProjLds::wt);
  constexpr int kNb = kColSlice / 8;
  constexpr int kPieces = (kKc / 4) * kNb;
  constexpr int kPer = kPieces / kDecThreads;
  static_assert(kPieces % kDecThreads == 0, "pieces split evenly");
  const __amdgpu_buffer_rsrc_t obuf = buffer_of(a.Wout, uint32_t(a.K) * a.d * 2);
  // One piece per thread at a time: the blocks of all projection
  // workgroups together are the whole of W_out, and issuing them in
  // batches keeps the memory queues short for the routing loads (measured:
  // with all batches in flight at once, every routing round waits behind
  // the W_out stream and the layer takes about 1.3 us longer).
  for (int u = 0; u < kPer; ++u) {
    const int c = threadIdx.x + u * kDecThreads;
    const int nb = c % kNb;
    const int kb = c / kNb;
    uint4 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = buffer_load16(obuf, uint32_t((kc * kKc + kb * 4 + i) * a.d + cs * kColSlice + nb * 8) * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint2 even = make_uint2(pack_lo(word(r[0], q), word(r[1], q)),
                                    pack_lo(word(r[2], q), word(r[3], q)));
      const uint2 odd = make_uint2(pack_hi(word(r[0], q), word(r[1], q)),
                                   pack_hi(word(r[2], q), word(r[3], q)));
      *reinterpret_cast<uint2*>(wt + (nb * 8 + 2 * q) * kWtPitch + kb * 4) = even;
      *reinterpret_cast<uint2*>(wt + (nb * 8 + 2 * q + 1) * kWtPitch + kb * 4) = odd;
    }
    // Keeps the compiler from hoisting the next batch's loads above these
    // stores (it would otherwise issue all of them at once).
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Partial product of item (kc, cs): partial[kc][t][cs*64 + c] (NaN when
// `poison`: the H it would read may be incomplete).  Wave w takes token
// block w (T <= 64) and all four 16-column groups.
__device__ void project_split(const DecodeArgs& a, unsigned char* lds, int kc, int cs,
                              bool poison) {
  const uint16_t* wt = reinterpret_cast<const uint16_t*>(lds + ProjLds::wt);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int n = lane & 15;  // column in a group (A row) / token in the block (B column)
  const int q = lane >> 4;
  const int tb = wave * 16;
  if (tb >= a.T) return;
  // Token columns past T are zero (no load).
  const __amdgpu_buffer_rsrc_t hbuf = buffer_of(a.H, uint32_t(a.T) * a.K * 2);
  const uint32_t hoff = uint32_t((tb + n) * a.K + kc * kKc + q * 8) * 2;
  uint4 hf[kKc / 32];
#pragma unroll
  for (int s = 0; s < kKc / 32; ++s) hf[s] = coherent_load16(hbuf, tb + n < a.T ? hoff + s * 64 : kOob);
  const __amdgpu_buffer_rsrc_t pbuf = buffer_of(a.partial, uint32_t(a.K / kKc) * a.T * a.d * 4);
#pragma unroll
  for (int cg = 0; cg < kColSlice / 16; ++cg) {
    const uint16_t* wrow = wt + (cg * 16 + n) * kWtPitch + q * 8;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < kKc / 32; ++s) {
      const uint4 wv = *reinterpret_cast<const uint4*>(wrow + s * 32);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv), as_bf16x8(hf[s]), acc, 0, 0, 0);
    }
    // acc[r]: column cg*16 + 4q + r, token tb + n.
    if (poison) acc = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                              __builtin_nanf("")};
    if (tb + n < a.T)
      coherent_store16(pbuf,
                       uint32_t((kc * a.T + tb + n) * a.d + cs * kColSlice + cg * 16 + q * 4) * 4,
                       make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                  __float_as_uint(acc[2]), __float_as_uint(acc[3])));
  }
}

// y columns of slice cs: sum of the K-chunk partials in chunk order.
__device__ void reduce_slice(const DecodeArgs& a, int cs) {
  const int nkc = a.K / kKc;
  const __amdgpu_buffer_rsrc_t pbuf = buffer_of(a.partial, uint32_t(nkc) * a.T * a.d * 4);
  for (int e = threadIdx.x; e < a.T * (kColSlice / 4); e += kDecThreads) {
    const int t = e / (kColSlice / 4);
    const int c = cs * kColSlice + (e - t * (kColSlice / 4)) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int kc = 0; kc < nkc; ++kc) {
      const uint4 v = coherent_load16(pbuf, uint32_t((kc * a.T + t) * a.d + c) * 4);
      s.x += __uint_as_float(v.x);
      s.y += __uint_as_float(v.y);
      s.z += __uint_as_float(v.z);
      s.w += __uint_as_float(v.w);
    }
    *reinterpret_cast<uint2*>(a.y + static_cast<int64_t>(t) * a.d + c) =
        make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
  }
}

// y columns of slice cs set to NaN for every token (poisoned header).
__device__ void nan_slice(const DecodeArgs& a, int cs) {
  const uint32_t qnan = 0x7FC07FC0u;  // two bf16 quiet NaNs
  for (int e = threadIdx.x; e < a.T * (kColSlice / 4); e += kDecThreads) {
    const int t = e / (kColSlice / 4);
    const int c = cs * kColSlice + (e - t * (kColSlice / 4)) * 4;
    *reinterpret_cast<uint2*>(a.y + static_cast<int64_t>(t) * a.d + c) = make_uint2(qnan, qnan);
  }
}

__global__ __launch_bounds__(kDecThreads, 2) void decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int last, waited;
  const int per_tree = (a.T + a.tok - 1) / a.tok;
  const int nroute = a.P * per_tree;
  const int g = blockIdx.x;
  const int nkc = a.K / kKc;
  const int ncs = a.d / kColSlice;

  // The call's epoch.
  uint64_t e = a.seed;
  bool poisoned = false;
  if (a.device_epoch) {
    const uint64_t h0 = __hip_atomic_load(a.hdr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t h1 = __hip_atomic_load(a.hdr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (h0 != 0 && h0 <= kEpochMask) {
      if (h1 == (h0 ^ kHdrValid)) {
        e = (h0 + 1) & kDeviceEpochMask;
        e = e ? e : 1;
      } else if (h1 == (h0 ^ kHdrPoison)) {
        poisoned = true;
      }
    }
  } else if (g == 0 && threadIdx.x == 0) {
    // Recorded for a later captured call; nothing in this call reads it.
    __hip_atomic_store(a.hdr, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.hdr + 1, e ^ kHdrValid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (g < a.n_route_wg) {
    if (poisoned) return;
    for (int it = g; it < nroute; it += a.n_route_wg) {
      const int p = it / per_tree;
      const int t0 = (it - p * per_tree) * a.tok;
      route_item(a, lds, it, p, t0, min(a.tok, a.T - t0), e);
    }
    return;
  }
  const int j = g - a.n_route_wg;
  const int nproj = nkc * ncs;
  for (int it = j; it < nproj; it += a.n_proj_wg) {
    const int kc = it % nkc;
    const int cs = it / nkc;
    if (poisoned) {
      if (kc == 0) nan_slice(a, cs);
      continue;
    }
    __syncthreads();  // LDS of a previous item is no longer read
    load_wout_block(a, lds, kc, cs);
    if (threadIdx.x < kWave) {
      // Routing items (consecutive ids) of the trees whose columns overlap
      // this K chunk.
      const int p_lo = kc * kKc / a.h;
      int p_hi = (kc * kKc + kKc - 1) / a.h;
      if (p_hi > a.P - 1) p_hi = a.P - 1;
      const bool ok =
          wait_slots(a.done, p_lo * per_tree, (p_hi - p_lo + 1) * per_tree, e, a.spin_limit);
      if (threadIdx.x == 0) waited = ok;
    }
    __syncthreads();
    const bool gave_up = !waited;
    project_split(a, lds, kc, cs, gave_up);
    // Arrival: store this chunk's slot once the partial stores have
    // completed, wait for that store, then read the slice's slots.  The
    // workgroup whose slot store completes last sees every slot set; more
    // than one may, and each then writes the same y values.  A captured call
    // reads every slice's slots: the workgroup that sees all of them set
    // stores the header (more than one may, with the same values).
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x < kWave) {
      if (threadIdx.x == 0)
        __hip_atomic_store(a.arrive + static_cast<int64_t>(cs) * nkc + kc,
                           e | (gave_up ? kGaveUp : 0), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      wait_vmcnt<0>();
      const int first = a.device_epoch ? 0 : cs * nkc;
      const int n = a.device_epoch ? ncs * nkc : nkc;
      bool ok_slice = true, ok_all = true, any_gave_up = false;
      for (int i = threadIdx.x; i < n; i += kWave) {
        const uint64_t v =
            __hip_atomic_load(a.arrive + first + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool set = (v & kEpochMask) == e;
        ok_all &= set;
        if ((first + i) / nkc == cs) ok_slice &= set;
        any_gave_up |= (v & kGaveUp) != 0;
      }
      ok_slice = __all(ok_slice);
      ok_all = __all(ok_all);
      any_gave_up = __any(any_gave_up);
      if (threadIdx.x == 0) {
        last = ok_slice;
        if (a.device_epoch && ok_all) {
          __hip_atomic_store(a.hdr, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(a.hdr + 1, e ^ (any_gave_up ? kHdrPoison : kHdrValid),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();
    if (last) reduce_slice(a, cs);
  }
}

struct DeviceInfo {
  int cus = 0, per_cu = 0;
  bool ready = false;
};

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

// Epochs of ordinary calls: a per-process counter started at a random point
// (so that words left by other processes do not match), each value passed
// through the SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014) so that the runs of consecutive
// epochs a captured call derives from one of them do not overlap those of
// the next.  61 random bits: a repeat within a process is vanishingly
// unlikely (the finaliser is a bijection of the 64-bit counter).
uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{[] {
    std::random_device rd;
    const uint64_t t = static_cast<uint64_t>(
        std::chrono::steady_clock::now().time_since_epoch().count());
    return (uint64_t(rd()) << 32) ^ uint64_t(rd()) ^ (t * 0x9E3779B97F4A7C15ull);
  }()};
  uint64_t z = counter.fetch_add(1, std::memory_order_relaxed);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (z & kDeviceEpochMask) | kHostEpochBit;
}

}  // namespace

bool decode_supported(const Dims& s) {
  // Every buffer the kernel addresses (one tree's W_node or V_node rows,
  // W_out, the workspace arrays) stays below 2^31 bytes.
  return s.dtype == 1 && s.T >= 1 && s.T <= 64 && s.d % 128 == 0 && s.d <= kMaxD &&
         s.h % 8 == 0 && s.h <= kMaxH && s.K % kKc == 0 && s.D + 1 <= kMaxLevels &&
         s.K * s.d < (int64_t(1) << 30);
}

// Tokens per routing item.  A round evaluates at most kMaxRows node rows:
// below n distinct current nodes it takes the deepest subtree with
// n (2^levels - 1) rows that fit, so with at most 2 tokens per item every
// round after the first covers 3 levels (a depth-6 walk takes 2 rounds, not
// the 4 of a 16-token item whose tokens spread over 16 nodes).  Items must
// also fit half of a 256-CU grid at once (a routing workgroup that loops
// over items serializes their rounds): 2 tokens while that holds, else 8,
// else 16.  Measured at d = 2048, P = 32, D = 6: T = 64 takes 31.5 us with
// 16 tokens per item, 30.5 us with 8 and 39 us with 4 (512 items, two per
// routing workgroup).
static int tokens_per_item(const Dims& s) {
  if (s.T <= 16 && int64_t(s.P) * ((s.T + 1) / 2) <= 256) return 2;
  if (int64_t(s.P) * ((s.T + 7) / 8) <= 256) return 8;
  return kDecTok;
}

size_t decode_workspace(const Dims& s) {
  const size_t items = size_t(s.P) * ((s.T + tokens_per_item(s) - 1) / tokens_per_item(s));
  return 256 + up256(items * 8) + up256(size_t(s.T) * s.K * 2) +
         up256(size_t(s.d / kColSlice) * (s.K / kKc) * 8) + up256(size_t(s.K / kKc) * s.T * s.d * 4);
}

hipError_t launch_decode(const Dims& s, const void* x, const void* W, const void* b,
                         const void* V, const void* Wout, void* y, int32_t* path_out, void* ws,
                         int flags, hipStream_t st) {
  DecodeArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.W = static_cast<const uint16_t*>(W);
  a.b = static_cast<const uint16_t*>(b);
  a.V = static_cast<const uint16_t*>(V);
  a.Wout = static_cast<const uint16_t*>(Wout);
  a.y = static_cast<uint16_t*>(y);
  a.path_out = path_out;
  a.tok = tokens_per_item(s);
  const int nroute = s.P * static_cast<int>((s.T + a.tok - 1) / a.tok);
  char* w = static_cast<char*>(ws);
  a.hdr = reinterpret_cast<uint64_t*>(w);
  w += 256;
  a.done = reinterpret_cast<uint64_t*>(w);
  w += up256(size_t(nroute) * 8);
  a.H = reinterpret_cast<uint16_t*>(w);
  w += up256(size_t(s.T) * s.K * 2);
  a.arrive = reinterpret_cast<uint64_t*>(w);
  w += up256(size_t(s.d / kColSlice) * (s.K / kKc) * 8);
  a.partial = reinterpret_cast<float*>(w);
  a.T = static_cast<int>(s.T);
  a.d = s.d;
  a.P = s.P;
  a.D = s.D;
  a.h = s.h;
  a.post = s.variant;
  a.alive = s.prune ? s.prune->alive : nullptr;
  a.K = static_cast<int>(s.K);
  a.N = s.N;

  // Per-device residency limit, queried once per device.
  static DeviceInfo info[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  DeviceInfo& di = info[dev];
  if (!di.ready) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(kDecLds));
    if (e == hipSuccess) e = hipDeviceGetAttribute(&di.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&di.per_cu, decode_kernel, kDecThreads, kDecLds);
    if (e != hipSuccess) return e;
    if (di.cus < 1 || di.per_cu < 1) return hipErrorInvalidConfiguration;
    di.ready = true;
  }
  // Grid no larger than what the device holds at once; items beyond it are
  // looped over.  Routing gets at most half of the slots.
  const int cap = di.cus * di.per_cu;
  const int nproj = static_cast<int>(s.K / kKc) * (s.d / kColSlice);
  a.n_route_wg = nroute < cap / 2 ? nroute : cap / 2;
  a.n_proj_wg = nproj < cap - a.n_route_wg ? nproj : cap - a.n_route_wg;
  if (a.n_proj_wg < 1) return hipErrorInvalidConfiguration;
  // A captured call takes its epoch from the workspace header (see above).
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(st, &capture);
  if (e != hipSuccess) return e;
  a.device_epoch = capture == hipStreamCaptureStatusActive ? 1 : 0;
  a.seed = next_epoch();
  const bool test_no_publish = (flags & FFF_PLAN_TEST_DECODE_NO_PUBLISH) != 0;
  a.publish = test_no_publish ? 0 : 1;
  a.spin_limit = test_no_publish ? kTestSpinLimit : kSpinLimit;
  hipLaunchKernelGGL(decode_kernel, dim3(a.n_route_wg + a.n_proj_wg), dim3(kDecThreads), kDecLds,
                     st, a);
  return hipGetLastError();
}

}  // namespace fff
