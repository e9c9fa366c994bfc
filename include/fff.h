/*
 * fff.h -- C ABI of the Fast FeedForward (FFF) layer forward pass on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation
 * -------------
 * "Dynamic sparsity in tree-structured feed-forward layers at scale": the
 * explainer page (gist.science, section 2, Methodology) describes an FFF
 * layer as P parallel perfect binary trees of depth D in which each token
 * follows one root-to-leaf path per tree, the sign of a per-node linear logit
 * choosing the branch, and only the visited nodes' outputs are summed; the
 * paper's own page (thelatestinai.com, Figure 1(c) caption) concatenates the
 * P tree outputs and applies one final linear projection; section 3.C of the
 * explainer puts the GELU before the summation.  With N = 2^(D+1) - 1 nodes
 * per tree, for every token x (a row of x[T,d]) and tree p:
 *
 *     n = 0 (root);  acc = 0 (h values)
 *     for level = 0 .. D:
 *         a    = x . W_node[p,n,:] + b_node[p,n]
 *         acc += GELU(a) * V_node[p,n,:]
 *         if level < D:  n = 2n+1 if a < 0 else 2n+2
 *     path_out[t,p] = n - (2^D - 1)            (leaf index)
 *     H[t, p*h : (p+1)*h] = acc
 *     y[t,:] = H[t,:] . W_out                  (no bias)
 *
 * Section 3.C of the explainer also describes FFF-post, in which the node
 * outputs are summed before the nonlinearity (the paper's page, Figure 3 and
 * Table 6, lists it beside FFF).  With shape->variant = FFF_VARIANT_POST the
 * loop above accumulates a * V_node[p,n,:] instead, and H[t, p*h + j] =
 * GELU(acc[j]) for each of the h elements; routing is unchanged.
 *
 * Readings fixed here where the pages are silent: GELU is the tanh form
 * 0.5 a (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))); a logit of exactly 0 (or
 * -0, or NaN) goes right; nodes are numbered in heap order; tree p owns
 * columns [p*h, (p+1)*h) of H and rows [p*h, (p+1)*h) of W_out; bit (D-1-l)
 * of a leaf index is the level-l decision, 1 = right.
 *
 * Layout and precision
 * --------------------
 * Every tensor is dense, row-major and of one dtype (FFF_DTYPE_F32 or
 * FFF_DTYPE_BF16):  x[T,d]  W_node[P,N,d]  b_node[P,N]  V_node[P,N,h]
 * W_out[P*h,d]  y[T,d].  path_out[T,P] is int32.  Logits, GELU and sums are
 * computed in fp32; for bf16 the concatenated tree outputs are rounded to
 * bf16 once (they feed the projection's matrix cores) and y is rounded to
 * bf16 (nearest even).
 *
 * Ownership, streams and errors
 * -----------------------------
 * All tensor and workspace pointers are device pointers owned by the caller.
 * The library allocates no memory and keeps no state between calls; calls
 * that use distinct workspaces may run concurrently.  Work is enqueued on
 * `stream` (0 = the null stream) and the call returns without waiting;
 * faults inside kernels surface at the caller's next synchronisation.
 * Arguments are validated on the host before any HIP call: on a validation
 * error nothing is enqueued.  Launch failures return FFF_ERROR_HIP.
 */
#ifndef FFF_H
#define FFF_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FFF_MAX_DEPTH 20

typedef enum fff_dtype {
    FFF_DTYPE_F32 = 0,
    FFF_DTYPE_BF16 = 1
} fff_dtype_t;

typedef enum fff_status {
    FFF_SUCCESS = 0,
    FFF_ERROR_INVALID_VALUE = 1, /* bad shape, null or misaligned pointer */
    FFF_ERROR_NOT_SUPPORTED = 2, /* unknown dtype, or a plan the shape cannot take */
    FFF_ERROR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    FFF_ERROR_HIP = 4            /* a HIP launch or runtime call failed */
} fff_status_t;

/* Where the GELU sits: on each visited node's logit before the node outputs
 * are summed (FFF), or on each element of the summed h-vector (FFF-post). */
typedef enum fff_variant {
    FFF_VARIANT_FFF = 0,
    FFF_VARIANT_POST = 1
} fff_variant_t;

/* Layer shape.  N = 2^(D+1) - 1 is implied.  Limits: T >= 0, d, P, h >= 1,
 * 0 <= D <= FFF_MAX_DEPTH, T < 2^31, and every tensor below 2^40 elements.
 * A variant other than those of fff_variant_t is FFF_ERROR_INVALID_VALUE;
 * every algorithm takes both variants. */
typedef struct fff_shape {
    int64_t T;       /* tokens */
    int32_t d;       /* model width */
    int32_t P;       /* parallel trees */
    int32_t D;       /* depth: D+1 nodes visited per path */
    int32_t h;       /* output width of one node */
    int32_t dtype;   /* fff_dtype_t */
    int32_t variant; /* fff_variant_t */
} fff_shape_t;

/* Algorithms.  AUTO picks by shape; the others force one (for tests and
 * measurement).  GENERIC takes any shape and dtype.  PREFILL needs bf16,
 * d % 64 == 0, h % 64 == 0 and either 2^(D+1) <= 256 (every level dense) or
 * a split level k with 1 <= k <= 8 and D-k <= 3 for the deep levels k..D:
 * through the token-tile kernel when k <= 5 and D <= 7, or bucketed when
 * d % 256 == 0, d <= 2048 and h <= 512.  AUTO evaluates every level densely
 * up to depth 5, the top D-3 levels densely and the last four per token tile
 * at depths 6 and 7, and buckets the last four from depth 8.  DECODE (one kernel for
 * the whole layer, routing overlapped with the stream of W_out) needs bf16,
 * 1 <= T <= 64, d % 128 == 0, d <= 2048, h % 8 == 0, h <= 256,
 * P*h % 512 == 0 and D <= 15; AUTO takes it whenever the shape allows.
 *
 * DECODE hands data between workgroups through slots in the workspace,
 * tagged with a per-call epoch; nothing needs clearing between calls.  An
 * ordinary call takes a fresh epoch from the host.  A call captured into a
 * HIP graph (the stream is capturing when fff_forward is called) takes its
 * epoch from a header word in the workspace instead: the call reads it at
 * entry and the last workgroup to finish advances it, so every replay gets a
 * new epoch.  Replays of one workspace must not overlap (one stream, or
 * ordered streams).  PREFILL and GENERIC plans launch only ordinary kernels
 * (no memset nodes) and capture as they are.
 *
 * DECODE assumes its workgroups are resident together (the grid is sized
 * from the device's occupancy); a workgroup that waits for another polls a
 * bounded number of times (about 0.1 s).  If a wait gives up, the columns
 * of y that depend on it come out NaN, for every token, and the kernel
 * still ends normally.  In a captured call a give-up also marks the
 * workspace header: every later captured call on that workspace then
 * writes NaN to all of y (and leaves path_out as it was), without waiting,
 * until an ordinary (uncaptured) DECODE call on the workspace, or clearing
 * the workspace's first 256 bytes, resets it. */
typedef enum fff_algo {
    FFF_ALGO_AUTO = 0,
    FFF_ALGO_GENERIC = 1,
    FFF_ALGO_PREFILL = 2,
    FFF_ALGO_DECODE = 3
} fff_algo_t;

typedef struct fff_plan {
    int32_t algo;         /* fff_algo_t */
    int32_t split_level;  /* PREFILL: levels 0..k-1 are evaluated as one dense
                             matrix product over all tokens; levels k..D (at
                             most 4 of them) per bucket of tokens sharing a
                             level-k node.  k = D+1 evaluates every level
                             densely.  -1 = choose by shape; ignored by other
                             algorithms */
    int32_t chunk_tokens; /* PREFILL with k <= D: 0 = the token-tile kernel
                             where the shape allows it (it stays 0 in the
                             resolved plan), else bucketing with a chunk
                             chosen by shape; > 0 = bucketing, in chunks of
                             this many tokens (a chunk's x rows are reread
                             from cache by all trees; each chunk restages
                             every subtree's rows) */
    int32_t flags;        /* 0, or FFF_PLAN_* bits below; other bits are
                             FFF_ERROR_INVALID_VALUE */
} fff_plan_t;

/* For tests of the decode wait's give-up only: DECODE's routing workgroups
 * do not publish their items, and the projection's waits poll a few times
 * instead of about 0.1 s, so every wait gives up and y comes out NaN (see
 * the DECODE notes above).  Other algorithms ignore it. */
#define FFF_PLAN_TEST_DECODE_NO_PUBLISH 1

/* Optional events recorded on `stream` at stage boundaries (each may be
 * NULL), in this order:
 *   start     before the first kernel
 *   prepared  with `start` (no plan prepares anything before routing: every
 *             projection kernel reads W_out in its own layout); kept so
 *             that the list of stages stays the same
 *   top       after the densely evaluated levels (GENERIC: every level's
 *             logits)
 *   deep      after the deep levels (the token-tile or bucketed kernels;
 *             with `top` where every level is dense)
 *   routed    once the concatenated tree outputs H are complete
 *   done      after the projection
 * A stage a plan does not have is recorded together with the previous
 * event; DECODE (one kernel for the whole layer) records `start` before it
 * and every other event after it.  The interval between two consecutive
 * events is that stage's time on the stream. */
typedef struct fff_stage_events {
    hipEvent_t start;
    hipEvent_t prepared;
    hipEvent_t top;
    hipEvent_t deep;
    hipEvent_t routed;
    hipEvent_t done;
} fff_stage_events_t;

/* Fill *plan with the choice FFF_ALGO_AUTO makes for this shape. */
fff_status_t fff_plan_default(const fff_shape_t *shape, fff_plan_t *plan);

/* Copy *in to *out with every 'choose by shape' field (algo AUTO,
 * split_level -1, chunk_tokens 0) replaced by the value the library would
 * use.  FFF_ERROR_NOT_SUPPORTED if the shape cannot run the requested plan. */
fff_status_t fff_plan_resolve(const fff_shape_t *shape, const fff_plan_t *in, fff_plan_t *out);

/* Workspace bytes the plan needs (plan NULL = the default plan), enough for
 * both fff_forward and fff_route under that plan.  The size depends only on
 * the shape and plan. */
fff_status_t fff_workspace_size(const fff_shape_t *shape, const fff_plan_t *plan, size_t *bytes);

/*
 * The whole layer: y = concat_p(tree outputs) . W_out, and path_out.
 *   x, W_node, b_node, V_node, W_out  inputs (device, dtype, 16-byte aligned
 *                                     except b_node: element aligned)
 *   y          output [T,d] (device, dtype, 16-byte aligned)
 *   path_out   output [T,P] int32 leaf indices, or NULL to skip
 *   workspace  device scratch of at least fff_workspace_size() bytes,
 *              256-byte aligned; may be NULL when that size is 0
 *   plan       NULL = default plan
 *   events     NULL = no events
 * T == 0 is a no-op that returns FFF_SUCCESS without touching any pointer.
 */
fff_status_t fff_forward(const fff_shape_t *shape, const fff_plan_t *plan,
                         const void *x, const void *W_node, const void *b_node,
                         const void *V_node, const void *W_out, void *y, int32_t *path_out,
                         void *workspace, size_t workspace_bytes, hipStream_t stream,
                         const fff_stage_events_t *events);

/*
 * Routing only: the concatenated tree outputs H[T, P*h] (dtype) and
 * path_out, without the projection.  Same rules as fff_forward; `H` is a
 * caller buffer (16-byte aligned).  Uses the same workspace size.  Runs a
 * staged algorithm: AUTO picks PREFILL or GENERIC, and DECODE (which fuses
 * the projection) returns FFF_ERROR_NOT_SUPPORTED.
 */
fff_status_t fff_route(const fff_shape_t *shape, const fff_plan_t *plan,
                       const void *x, const void *W_node, const void *b_node,
                       const void *V_node, void *H, int32_t *path_out,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Projection only: y[T,d] = H[T,K] . W_out[K,d] with K = P*h, fp32
 * accumulation, output rounded to dtype.  `algo` selects the kernel family
 * (AUTO, GENERIC, or PREFILL for the matrix-core kernels; where the
 * direct-to-LDS product applies (bf16, K % 32 == 0 and at least 256 output
 * tiles of 256 x 256 or 128 x 128) it is the kernel fff_forward uses for its
 * projection, so y equals fff_forward's y for the same H).  Needs no
 * workspace.
 */
fff_status_t fff_project(const fff_shape_t *shape, int32_t algo, const void *H,
                         const void *W_out, void *y, hipStream_t stream);

/*
 * Workspace bytes of fff_project_ws for this shape and algo: always 0 (no
 * projection kernel needs workspace).  `bytes` must not be NULL.  Same
 * shape and algo rules as fff_project.
 */
fff_status_t fff_project_workspace_size(const fff_shape_t *shape, int32_t algo, size_t *bytes);

/*
 * fff_project with a caller workspace, which no kernel uses any more
 * (fff_project_workspace_size() is 0; the workspace may be NULL): the same
 * kernels and results as fff_project.  The product is the layer's final
 * linear projection of the concatenated tree outputs (the paper's page,
 * Figure 1(c) caption).
 */
fff_status_t fff_project_ws(const fff_shape_t *shape, int32_t algo, const void *H,
                            const void *W_out, void *y, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * Static path pruning
 * -------------------
 * The paper's page (Figure 4) removes paths of trained trees permanently at
 * fixed ratios, and the explainer page (section 3.B) describes paths that
 * training itself leaves inactive.  Here a mask marks each leaf (path) of
 * each tree alive or pruned; a node is alive when some leaf below it is.
 * The pages do not say where a token goes when its logit points into a
 * pruned subtree: it takes the other child, which is alive whenever its
 * parent is.  Every tree must keep at least one alive leaf.  Routing,
 * nonlinearity and projection are otherwise those of fff_forward.
 *
 * The mask is static, so it is prepared once into a device table owned by
 * the caller: node alive flags, and for the PREFILL plan the alive node rows
 * of the densely evaluated levels (< split_level) packed tree by tree into
 * 256-column tiles, so that the dense product reads and multiplies only
 * those.  The packed rows are a copy of W_node: prepare again after the
 * weights change.
 */
typedef struct fff_pruning {
    const void *table;   /* device table written by fff_prune_prepare */
    int32_t P, D, d;     /* the shape it was prepared for */
    int32_t split_level; /* PREFILL split level whose rows are packed; 0 = none */
    int32_t col_tiles;   /* 256-column tiles of packed rows (at least 1 when
                            split_level > 0; a table whose fields do not fit
                            the shape is FFF_ERROR_INVALID_VALUE) */
} fff_pruning_t;

/* Device bytes of the table for this shape and plan (plan NULL = the
 * default plan; only the resolved algorithm and split level matter, T does
 * not once the plan is fixed). */
fff_status_t fff_prune_table_size(const fff_shape_t *shape, const fff_plan_t *plan, size_t *bytes);

/*
 * Builds the table.  leaf_alive: HOST array [P, 2^D] of bytes, nonzero =
 * alive.  W_node: the layer's node weights (device).  table: device buffer of
 * at least fff_prune_table_size() bytes, 256-byte aligned.  The call returns
 * once the table is complete on the device (it synchronizes `stream`), and
 * fills *out.  FFF_ERROR_INVALID_VALUE if a tree has no alive leaf or a
 * pointer is missing; FFF_ERROR_WORKSPACE if the table is too small.
 */
fff_status_t fff_prune_prepare(const fff_shape_t *shape, const fff_plan_t *plan,
                               const uint8_t *leaf_alive, const void *W_node, void *table,
                               size_t table_bytes, hipStream_t stream, fff_pruning_t *out);

/*
 * fff_forward on pruned trees.  Same arguments and workspace as fff_forward
 * plus the prepared table.  The plan resolves as for fff_forward; a PREFILL
 * plan must have the split level the table was prepared with
 * (FFF_ERROR_NOT_SUPPORTED otherwise); DECODE and GENERIC use the alive
 * flags only.  A table prepared for another P, D or d is
 * FFF_ERROR_INVALID_VALUE.
 */
fff_status_t fff_forward_pruned(const fff_shape_t *shape, const fff_plan_t *plan,
                                const fff_pruning_t *pruning, const void *x, const void *W_node,
                                const void *b_node, const void *V_node, const void *W_out,
                                void *y, int32_t *path_out, void *workspace,
                                size_t workspace_bytes, hipStream_t stream,
                                const fff_stage_events_t *events);

/*
 * Backward pass
 * -------------
 * Gradients of f = sum over t, c of y[t,c] * dy[t,c] with every token's
 * paths held as the forward pass takes them: the sign decision has no
 * gradient (the pages name no estimator) and only visited nodes receive one
 * (explainer page, section 3.B).  Per token t, tree p and visited node n
 * with logit a, dH = dy . W_out^T:
 *   FFF       da = GELU'(a) (dH_p . v_n),           dV_n += GELU(a) dH_p
 *   FFF-post  s = sum over the path of a v_n,      ds = GELU'(s) * dH_p,
 *             da = ds . v_n,                        dV_n += a ds
 *   db_n += da,  dW_n += da x_t,  dx_t += da w_n,   dW_out = H^T dy
 * (GELU' of the tanh form).  Pruned trees: fff_backward_pruned, below.
 *
 *   dy        [T,d] dtype (device)
 *   dx        [T,d] dtype out
 *   dW_node   [P,N,d] float32 out    db_node [P,N] float32 out
 *   dV_node   [P,N,h] float32 out    dW_out  [P*h,d] float32 out
 * Every output is overwritten (nodes off every path get 0).  Plans: GENERIC
 * (any shape and dtype) or PREFILL (bf16, every level dense: 3 <= D+1 <= 8,
 * d % 64 == 0, h % 64 == 0, P*2^(D+1) % 64 == 0, and one tree's v rows plus
 * 2^(D+1) floats within 64 KB); AUTO picks PREFILL when the
 * shape allows; DECODE and split PREFILL plans are FFF_ERROR_NOT_SUPPORTED.
 * Sums over tokens use float32 atomics in some kernels, so results may
 * differ in the last bits between calls.  Workspace: fff_backward_workspace_size.
 */
fff_status_t fff_backward_workspace_size(const fff_shape_t *shape, const fff_plan_t *plan,
                                         size_t *bytes);
fff_status_t fff_backward(const fff_shape_t *shape, const fff_plan_t *plan, const void *x,
                          const void *W_node, const void *b_node, const void *V_node,
                          const void *W_out, const void *dy, void *dx, float *dW_node,
                          float *db_node, float *dV_node, float *dW_out, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * fff_backward on pruned trees (paper page, Figure 4: paths removed
 * permanently): the same gradients with every token's paths as
 * fff_forward_pruned takes them, a routed step into a subtree with no alive
 * leaf going to the sibling.  Only visited nodes receive gradient (explainer
 * page, section 3.B), so every pruned node's dW_node, db_node and dV_node
 * come out 0.  Arguments, layouts, ownership and error codes as for
 * fff_backward, plus the table fff_prune_prepare built for these trees (one
 * prepared for another P, D or d is FFF_ERROR_INVALID_VALUE).  Plans: GENERIC
 * takes any table; PREFILL needs a table prepared with every level dense
 * (plan PREFILL, split_level D + 1), FFF_ERROR_NOT_SUPPORTED otherwise; AUTO
 * picks PREFILL when the shape and the table allow it.  Workspace:
 * fff_backward_pruned_workspace_size with the same plan and table.
 */
fff_status_t fff_backward_pruned_workspace_size(const fff_shape_t *shape, const fff_plan_t *plan,
                                                const fff_pruning_t *pruning, size_t *bytes);
fff_status_t fff_backward_pruned(const fff_shape_t *shape, const fff_plan_t *plan,
                                 const fff_pruning_t *pruning, const void *x, const void *W_node,
                                 const void *b_node, const void *V_node, const void *W_out,
                                 const void *dy, void *dx, float *dW_node, float *db_node,
                                 float *dV_node, float *dW_out, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  fff_forward with the library's own fixed scratch region as
 * the workspace: a device array of FFF_STATIC_SCRATCH_BYTES bytes that each
 * GPU the library runs on holds from the first call until the process ends.
 * The caller passes inputs and outputs as for fff_forward; the call makes no
 * allocation of any kind.
 *
 * Shapes whose fff_workspace_size() exceeds FFF_STATIC_SCRATCH_BYTES return
 * FFF_ERROR_WORKSPACE before any HIP call (so do the other validation
 * errors of fff_forward).  Every call on one GPU uses the same region and
 * leaves its contents behind; nothing in it needs to start at zero.  Calls
 * that overlap on one GPU (concurrent streams or host threads) race on it
 * and must be serialized by the caller.
 */
#define FFF_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
fff_status_t fff_forward_static(const fff_shape_t *shape, const fff_plan_t *plan,
                                const void *x, const void *W_node, const void *b_node,
                                const void *V_node, const void *W_out, void *y,
                                int32_t *path_out, hipStream_t stream,
                                const fff_stage_events_t *events);

/* Static, human-readable text for a status code. */
const char *fff_status_string(fff_status_t status);

/* Static name of an algorithm ("auto", "generic", "prefill", "decode"). */
const char *fff_algo_name(int32_t algo);

#ifdef __cplusplus
}
#endif

#endif /* FFF_H */
