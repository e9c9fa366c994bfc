// Host-side launchers of the gfx950 kernels.  Each enqueues its kernel(s) on
// `stream` and returns hipGetLastError().  Shapes have been validated by the
// C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <utility>
#include <vector>

namespace fff {

// Raises a kernel's dynamic-LDS limit to `bytes`, once per (kernel, device):
// the attribute belongs to the device current at the call.
inline hipError_t ensure_lds_limit(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& kd : done)
    if (kd.first == kernel && kd.second == dev) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.emplace_back(kernel, dev);
  return e;
}

// Static path pruning: views into a device table built once per leaf mask.
// A node is alive when some leaf below it is; a routed step into a pruned
// child goes to its sibling.  For the dense top levels the table also holds
// the alive node rows of levels < L packed tree by tree into 256-column
// tiles (no tree straddles a tile), so the dense product streams only them.
struct PruneView {
  const uint8_t* alive;        // [P][N] 1 = alive
  const int32_t* tree_base;    // [P] first packed column of tree p within its tile
  const int32_t* tile_first;   // [col_tiles] first tree of each tile
  const int32_t* tile_count;   // [col_tiles] trees in each tile
  const int32_t* colmap;       // [col_tiles * 256] heap row p*N + n of each packed column, -1 none
  const uint32_t* colinfo;     // [col_tiles * 256] children of each packed column: bits 0-8 and
                               // 9-17 their tile columns (dense levels), bits 18 / 19 alive
  const uint16_t* W_packed;    // [col_tiles * 256][d] packed rows (zero rows fill a tile)
  int L;                       // dense levels packed (0: none)
  int col_tiles;
};

struct Dims {
  int64_t T;
  int d, P, D, h;
  int dtype;    // fff_dtype_t
  int variant;  // fff_variant_t: 0 = GELU per node, 1 = GELU after the sum
  int64_t N;    // 2^(D+1) - 1
  int64_t K;    // P * h
  size_t esize;
  const PruneView* prune;  // null: every path alive
};

// ---- generic path: any shape, fp32 or bf16 ----
// Per (token, tree) logits of the visited nodes -> logits[T,P,D+1] (fp32) and
// path_out (may be null).
hipError_t launch_route_generic(const Dims& s, const void* x, const void* W, const void* b,
                                float* logits, int32_t* path_out, int32_t* leaf_ws,
                                hipStream_t st);
// H[t, p*h + j] = sum over levels of GELU(a_l) * V[p, n_l, j]  (variant 0), or
// GELU(sum over levels of a_l * V[p, n_l, j])  (variant 1).
hipError_t launch_hbuild_generic(const Dims& s, const float* logits, const int32_t* leaf_ws,
                                 const void* V, void* H, hipStream_t st);
// y = H . W_out with fp32 accumulation.
hipError_t launch_project_generic(const Dims& s, const void* H, const void* Wout, void* y,
                                  hipStream_t st);

// ---- matrix-core projection (bf16, K % 64 == 0, d % 64 == 0) ----
bool project_mfma_supported(const Dims& s);
hipError_t launch_project_mfma(const Dims& s, const void* H, const void* Wout, void* y,
                               hipStream_t st);

// Multi-stage direct-to-LDS projection (W_out in its own [K][d] layout; H
// row-major, or K-blocked as launch_hbuild writes it with `h_blocked`).
bool project_direct_supported(const Dims& s);
hipError_t launch_project_direct(const Dims& s, const void* H, const void* Wout, void* y,
                                 bool h_blocked, hipStream_t st);

// ---- prefill routing (bf16) ----
// Dense evaluation of tree levels 0..L-1 (L <= 8) with the walk over them:
// rec_logit[p][t][l] (fp32, record stride `stride` >= L floats) and
// rec_next[p][t] (heap id at level L, or the leaf when L = D+1).
bool route_top_supported(const Dims& s, int L);
hipError_t launch_route_top(const Dims& s, int L, int stride, const void* x, const void* W,
                            const void* b, float* rec_logit, int32_t* rec_next, hipStream_t st);
// H and path_out need the whole path's records (L = D+1 levels, stride D+1).
bool hbuild_supported(const Dims& s);
// H and path_out from fully routed records (L = D+1).  H row-major
// [T][K], or, with `blocked` (K % 32 == 0), K-blocked: element (t, k) at
// ((k / 32) * T + t) * 32 + k % 32, so that the 32-column K slice of a
// token tile is contiguous for the projection.
hipError_t launch_hbuild(const Dims& s, const float* rec_logit, const int32_t* rec_next,
                         const void* V, void* H, int32_t* path_out, bool blocked,
                         hipStream_t st);

// Dense levels 0..L-1 as two K halves of raw fp32 logits, for the
// token-tile plans of shapes with few column tiles (no walk: the token-tile
// kernel below takes the halves).  part holds route_top_split_bytes():
// part[(half * ncols + col) * T + t], ncols = route_top_split_cols().
bool route_top_split_wanted(const Dims& s, int L);
size_t route_top_split_bytes(const Dims& s, int L);
int route_top_split_cols(const Dims& s, int L);
hipError_t launch_route_top_split(const Dims& s, int L, const void* x, const void* W,
                                  float* part, hipStream_t st);

// Deep levels k..D per token tile (bf16; D-k <= 3, 1 <= k <= 5): for each
// token and tree, the 16-node block of its own level-k subtree on the matrix
// cores; completes rec_logit (levels k..D, stride D+1) and rec_next (leaf).
// With `part` (launch_route_top_split's halves, ncols columns) it first
// sums, biases and walks levels 0..k-1 itself and records them too; else it
// starts from rec_next (the level-k node).
bool subtree_supported(const Dims& s, int k);
hipError_t launch_subtree(const Dims& s, int k, const void* x, const void* W, const void* b,
                          float* rec_logit, int32_t* rec_next, const float* part, int ncols,
                          hipStream_t st);

// Deep levels k..D per token bucket (bf16; D-k <= 3).
bool deep_supported(const Dims& s, int k);
size_t deep_chunk(const Dims& s, int k);  // default tokens per bucket chunk
size_t bucket_count_bytes(const Dims& s, int k, int chunk);  // per-slice bucket counts
hipError_t launch_bucket(const Dims& s, int k, const int32_t* rec_next, int32_t* perm,
                         int32_t* offs, int32_t* cnt, int chunk, hipStream_t st);
hipError_t launch_deep(const Dims& s, int k, const void* x, const void* W, const void* b,
                       const void* V, const float* rec_logit, const int32_t* perm,
                       const int32_t* offs, void* H, int32_t* path_out, int chunk,
                       hipStream_t st);

// Copies the node rows that colmap[i] names (heap row p*N + n, or -1 for a
// zero row) into packed[i], for i < rows.
hipError_t launch_prune_pack(const void* W, const int32_t* colmap, void* packed, int rows, int d,
                             hipStream_t st);

// ---- decode (bf16, 1 <= T <= 64): one kernel for the whole layer ----
// Workspace: an epoch header, per-item and per-partial slots, H [T,K] bf16
// and fp32 K-chunk partials of y.  `flags`: fff_plan_t flags.
bool decode_supported(const Dims& s);
size_t decode_workspace(const Dims& s);
hipError_t launch_decode(const Dims& s, const void* x, const void* W, const void* b,
                         const void* V, const void* Wout, void* y, int32_t* path_out, void* ws,
                         int flags, hipStream_t st);

// ---- backward pass (gradients of sum(y * dy), paths held fixed) ----
hipError_t launch_fill_f32(float* p, int64_t n, hipStream_t st);
// Generic: any shape and dtype.  Uses the routing records of
// launch_route_generic; dW, db, dV, dWout are fp32 outputs; dH, Hf ([T,K])
// and dxacc ([T,d]) fp32 scratch.
hipError_t launch_backward_generic(const Dims& s, const void* x, const void* W, const void* V,
                                   const void* Wout, const void* dy, void* dx, float* dW, float* db,
                                   float* dV, float* dWout, const float* logits,
                                   const int32_t* leaf, float* dH, float* Hf, float* dxacc,
                                   hipStream_t st);

// Matrix-core path: bf16, every level dense (3 <= D+1 <= 8), d and h
// multiples of 64.  Workspace: routing records, transposed x and dy, dH, the
// masked DA (and its transpose), G^T, H^T, dS^T, the node rows transposed
// and the float32 partial products of the split token dimension.
struct BwdMfmaLayout {
  size_t logits, next, xT, dyT, dH, DA, DAt, Gt, Ht, dSt, WTn, part, total;
  int64_t Tp;  // tokens padded to a multiple of 256
};
bool backward_mfma_supported(const Dims& s);
BwdMfmaLayout backward_mfma_layout(const Dims& s);
hipError_t launch_backward_mfma(const Dims& s, const void* x, const void* W, const void* b,
                                const void* V, const void* Wout, const void* dy, void* dx,
                                float* dW, float* db, float* dV, float* dWout, void* ws,
                                hipStream_t st);

}  // namespace fff
