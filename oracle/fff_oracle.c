/*
 * fff_oracle.c -- plain CPU reference for the Fast FeedForward (FFF) layer
 * forward and backward passes.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the HIP library never does, and
 * the two share no code.
 *
 * Everything is float64.  Inputs arrive already widened (exactly) to double.
 * Loops run in the plain textbook order (i ascending in every dot product).
 *
 * What is computed, and where it is stated:
 *
 *  - "Dynamic sparsity in tree-structured feed-forward layers at scale"
 *    (gist.science explainer, section 2, Methodology): P parallel perfect
 *    binary trees of depth D; per token one root-to-leaf path per tree; at
 *    every node a linear projection of the input gives a logit whose sign
 *    picks the child; only the nodes on the path are evaluated and their
 *    outputs are summed.
 *  - Same page, section 3.C: two placements of the nonlinearity.  In FFF
 *    (variant 0) GELU is applied per node, before the node outputs are
 *    summed; in FFF-post (variant 1) the node outputs a_n * v_n are summed
 *    first and GELU is applied once to each element of the tree's h-vector.
 *    The thelatestinai.com page, Figure 3 and Table 6, names both variants.
 *    Routing is the same in both: it depends on the logits only.
 *  - thelatestinai.com page of the same paper, Figure 1(c) caption: the tree
 *    outputs are concatenated and passed through one final linear projection.
 *  - Table 4 of that page (MLP-block sparsity 83% / 94% / 99% at depths
 *    4 / 6 / 13) matches D+1 evaluated nodes out of 2^(D+1)-1, so every node
 *    on the path, leaf included, contributes.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes):  node n computes a = x.w_n + b_n and contributes GELU(a) * v_n,
 * v_n in R^h;  GELU is the tanh form 0.5 a (1 + tanh(sqrt(2/pi)(a + 0.044715
 * a^3)));  a < 0 goes to the left child, anything else (0, -0, NaN) to the
 * right;  nodes are numbered in heap order (children of n: 2n+1 left, 2n+2
 * right);  tree p fills columns [p*h, (p+1)*h) of the concatenation and rows
 * [p*h, (p+1)*h) of W_out;  there is no projection bias;  path_out holds the
 * leaf index n - (2^D - 1), whose bit (D-1-l) is the level-l decision
 * (1 = right).
 *
 * Static path pruning (thelatestinai.com page, Figure 4: paths removed
 * permanently at fixed ratios; explainer page, section 3.B: paths that
 * training leaves inactive): an optional mask marks each leaf of each tree
 * alive or pruned.  A node is alive when some leaf below it is alive.  The
 * pages do not say where a token goes when its logit points into a pruned
 * subtree; here it takes the other child, which is alive whenever its parent
 * is.  Every tree must keep at least one alive leaf.
 *
 * Near-tie threshold: for each visited node the oracle also records
 * thr = 1e-4 * ||x_t||_2 * ||w_n||_2; a device path that takes the other
 * branch at a node whose |a| <= thr is excused (and counted) by the tests.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define FFFO_OK 0
#define FFFO_BAD_ARG 1

static double gelu_tanh(double a)
{
    const double k0 = 0.7978845608028654; /* sqrt(2/pi) */
    const double k1 = 0.044715;
    return 0.5 * a * (1.0 + tanh(k0 * (a + k1 * a * a * a)));
}

static double dot(const double *u, const double *v, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i)
        s += u[i] * v[i];
    return s;
}

/*
 * alive[0..N) of one tree from its leaf mask (leaf i is heap node 2^D-1+i):
 * leaves as given, every internal node alive iff one of its children is.
 */
static void alive_nodes(const uint8_t *leaf_alive, int D, uint8_t *alive)
{
    const int64_t first_leaf = ((int64_t)1 << D) - 1;
    for (int64_t i = 0; i <= first_leaf; ++i)
        alive[first_leaf + i] = leaf_alive[i] != 0;
    for (int64_t n = first_leaf - 1; n >= 0; --n)
        alive[n] = alive[2 * n + 1] | alive[2 * n + 2];
}

/*
 * One token through one tree.  Walks root to leaf, adding GELU(a) * v_n
 * (variant 0) or a * v_n (variant 1) for every visited node into acc[0..h);
 * variant 1 then replaces each acc[j] by GELU(acc[j]).  If forced_leaf >= 0
 * the branch at each level is taken from that leaf's bits instead of the
 * logit's sign.  With `alive` (this tree's node mask, or NULL for an
 * unpruned tree) a routed step into a pruned child goes to its sibling.
 * Returns the leaf index.
 */
static int32_t walk_tree(const double *xt, double xnorm, const double *Wp, const double *bp,
                         const double *Vp, int d, int D, int h, int variant, int32_t forced_leaf,
                         const uint8_t *alive, double *acc, double *rec_a, double *rec_thr, int32_t *rec_node)
{
    int64_t n = 0; /* heap index of the current node */
    for (int j = 0; j < h; ++j)
        acc[j] = 0.0;
    for (int level = 0; level <= D; ++level) {
        const double *w = Wp + n * (int64_t)d;
        double a = dot(xt, w, d) + bp[n];
        if (rec_a)
            rec_a[level] = a;
        if (rec_thr)
            rec_thr[level] = 1e-4 * xnorm * sqrt(dot(w, w, d));
        if (rec_node)
            rec_node[level] = (int32_t)n;
        double g = variant == 1 ? a : gelu_tanh(a);
        const double *v = Vp + n * (int64_t)h;
        for (int j = 0; j < h; ++j)
            acc[j] += g * v[j];
        if (level < D) {
            int go_right;
            if (forced_leaf >= 0)
                go_right = (forced_leaf >> (D - 1 - level)) & 1;
            else {
                go_right = !(a < 0.0);
                if (alive && !alive[2 * n + 1 + go_right])
                    go_right = !go_right;
            }
            n = 2 * n + 1 + go_right;
        }
    }
    if (variant == 1)
        for (int j = 0; j < h; ++j)
            acc[j] = gelu_tanh(acc[j]);
    return (int32_t)(n - (((int64_t)1 << D) - 1));
}

/*
 * fffo_forward: the whole layer for T tokens.
 *
 *   x [T,d], W [P,N,d], b [P,N], V [P,N,h], Wout [P*h,d]   (N = 2^(D+1)-1)
 *   forced  [T,P] leaf indices, or NULL to route by sign
 *   leaf_alive  [P, 2^D] nonzero = alive, or NULL for unpruned trees; a tree
 *               with no alive leaf is a bad argument
 *   y       [T,d] out, or NULL to skip the projection
 *   H       [T,P*h] out (the concatenated tree outputs), or NULL
 *   path    [T,P] out (leaf indices), or NULL
 *   rec_a, rec_thr, rec_node  [T,P,D+1] per-visit records, each may be NULL
 *   variant   0 = FFF (GELU per node), 1 = FFF-post (GELU after the sum)
 *   nthreads  worker threads (<= 0: runtime default)
 *
 * Returns 0, or 1 for a bad shape or variant.
 */
int fffo_forward(int64_t T, int d, int P, int D, int h, int variant,
                 const double *x, const double *W, const double *b, const double *V,
                 const double *Wout, const int32_t *forced, const uint8_t *leaf_alive,
                 double *y, double *H, int32_t *path,
                 double *rec_a, double *rec_thr, int32_t *rec_node, int nthreads)
{
    if (T < 0 || d <= 0 || P <= 0 || D < 0 || D > 24 || h <= 0 || variant < 0 || variant > 1)
        return FFFO_BAD_ARG;
    const int64_t N = ((int64_t)1 << (D + 1)) - 1;
    const int64_t K = (int64_t)P * h;
    const int L = D + 1;
    if (nthreads <= 0)
        nthreads = 1;
    uint8_t *alive = NULL;
    if (leaf_alive) {
        alive = (uint8_t *)malloc((size_t)(P * N));
        if (!alive)
            abort();
        for (int p = 0; p < P; ++p) {
            alive_nodes(leaf_alive + ((int64_t)p << D), D, alive + p * N);
            if (!alive[p * N]) {
                free(alive);
                return FFFO_BAD_ARG;
            }
        }
    }

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t t = 0; t < T; ++t) {
        const double *xt = x + t * d;
        double xnorm = sqrt(dot(xt, xt, d));
        double *Ht = (double *)malloc(sizeof(double) * (size_t)K);
        if (!Ht)
            abort();
        for (int p = 0; p < P; ++p) {
            int64_t tp = t * P + p;
            int32_t fl = forced ? forced[tp] : -1;
            int32_t leaf = walk_tree(xt, xnorm, W + (int64_t)p * N * d, b + (int64_t)p * N,
                                     V + (int64_t)p * N * h, d, D, h, variant, fl,
                                     alive ? alive + p * N : NULL, Ht + (int64_t)p * h,
                                     rec_a ? rec_a + tp * L : NULL,
                                     rec_thr ? rec_thr + tp * L : NULL,
                                     rec_node ? rec_node + tp * L : NULL);
            if (path)
                path[tp] = leaf;
        }
        if (H)
            for (int64_t k = 0; k < K; ++k)
                H[t * K + k] = Ht[k];
        if (y) {
            /* y[t,c] = sum over k ascending of H[t,k] * Wout[k,c]; the k loop
             * is outermost only so that Wout is read row by row. */
            double *yt = y + t * d;
            for (int c = 0; c < d; ++c)
                yt[c] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double hk = Ht[k];
                const double *wk = Wout + k * d;
                for (int c = 0; c < d; ++c)
                    yt[c] += hk * wk[c];
            }
        }
        free(Ht);
    }
    free(alive);
    return FFFO_OK;
}

/*
 * Backward pass.  The paths are those of the forward pass (hard decisions,
 * no gradient through them: explainer page, section 3.B, describes
 * gradients that reach only the visited nodes); every visited node's output
 * is differentiated with the routing held fixed.  With f the scalar
 * sum over t, c of y[t,c] * dy[t,c]:
 *
 *   dH[t,k]        = sum_c dy[t,c] Wout[k,c]
 *   dWout[k,c]     = sum_t H[t,k] dy[t,c]
 *   FFF (variant 0), per visited node n at level l of tree p:
 *     da           = GELU'(a) * sum_j dH[t, p*h+j] V[p,n,j]
 *     dV[p,n,j]   += GELU(a) * dH[t, p*h+j]
 *   FFF-post (variant 1), with s_j = sum over the path of a * V[p,n,j]:
 *     ds_j         = GELU'(s_j) * dH[t, p*h+j]
 *     da           = sum_j ds_j V[p,n,j]
 *     dV[p,n,j]   += a * ds_j
 *   then  db[p,n] += da;  dW[p,n,:] += da * x[t,:];  dx[t,:] += da * W[p,n,:].
 *
 * GELU'(a) of the tanh form, u = sqrt(2/pi)(a + 0.044715 a^3):
 *   0.5 (1 + tanh u) + 0.5 a (1 - tanh^2 u) sqrt(2/pi) (1 + 3 * 0.044715 a^2).
 *
 * Outputs (all float64, fully overwritten): dx [T,d], dW [P,N,d], db [P,N],
 * dV [P,N,h], dWout [P*h,d].  Sums over tokens run in ascending t.
 * Returns 0, or 1 for a bad argument (as fffo_forward).
 */
static double gelu_tanh_grad(double a)
{
    const double k0 = 0.7978845608028654;
    const double k1 = 0.044715;
    const double th = tanh(k0 * a * (1.0 + k1 * a * a));
    return 0.5 * (1.0 + th) + 0.5 * a * (1.0 - th * th) * k0 * (1.0 + 3.0 * k1 * a * a);
}

int fffo_backward(int64_t T, int d, int P, int D, int h, int variant,
                  const double *x, const double *W, const double *b, const double *V,
                  const double *Wout, const uint8_t *leaf_alive, const double *dy,
                  double *dx, double *dW, double *db, double *dV, double *dWout, int nthreads)
{
    if (T < 0 || d <= 0 || P <= 0 || D < 0 || D > 24 || h <= 0 || variant < 0 || variant > 1)
        return FFFO_BAD_ARG;
    const int64_t N = ((int64_t)1 << (D + 1)) - 1;
    const int64_t K = (int64_t)P * h;
    const int L = D + 1;
    if (nthreads <= 0)
        nthreads = 1;
    uint8_t *alive = NULL;
    if (leaf_alive) {
        alive = (uint8_t *)malloc((size_t)(P * N));
        if (!alive)
            abort();
        for (int p = 0; p < P; ++p) {
            alive_nodes(leaf_alive + ((int64_t)p << D), D, alive + p * N);
            if (!alive[p * N]) {
                free(alive);
                return FFFO_BAD_ARG;
            }
        }
    }
    /* Forward records (the forward walk itself): visited nodes and logits
     * [T,P,L], H [T,K], and for FFF-post the summed pre-activation S [T,K]. */
    int32_t *node = (int32_t *)calloc((size_t)(T * P * L + 1), sizeof(int32_t));
    double *la = (double *)calloc((size_t)(T * P * L + 1), sizeof(double));
    double *H = (double *)malloc(sizeof(double) * (size_t)(T * K + 1));
    double *S = (double *)malloc(sizeof(double) * (size_t)(T * K + 1));
    double *dH = (double *)malloc(sizeof(double) * (size_t)(T * K + 1));
    double *da = (double *)malloc(sizeof(double) * (size_t)(T * P * L + 1));
    if (!node || !la || !H || !S || !dH || !da)
        abort();

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t t = 0; t < T; ++t) {
        const double *xt = x + t * d;
        for (int p = 0; p < P; ++p) {
            const double *Vp = V + (int64_t)p * N * h;
            const int64_t tp = t * P + p;
            walk_tree(xt, 0.0, W + (int64_t)p * N * d, b + (int64_t)p * N, Vp, d, D, h, variant,
                      -1, alive ? alive + p * N : NULL, H + t * K + (int64_t)p * h,
                      la + tp * L, NULL, node + tp * L);
            double *St = S + t * K + (int64_t)p * h;
            for (int j = 0; j < h; ++j) {
                St[j] = 0.0;
                for (int level = 0; level <= D; ++level)
                    St[j] += la[tp * L + level] * Vp[(int64_t)node[tp * L + level] * h + j];
            }
        }
        /* dH, then da and dx for this token. */
        const double *dyt = dy + t * d;
        for (int64_t k = 0; k < K; ++k)
            dH[t * K + k] = dot(dyt, Wout + k * d, d);
        double *dxt = dx + t * d;
        for (int c = 0; c < d; ++c)
            dxt[c] = 0.0;
        for (int p = 0; p < P; ++p) {
            const double *Vp = V + (int64_t)p * N * h;
            const double *dHp = dH + t * K + (int64_t)p * h;
            const double *Sp = S + t * K + (int64_t)p * h;
            const int64_t tp = t * P + p;
            for (int level = 0; level <= D; ++level) {
                const int64_t n = node[tp * L + level];
                double g = 0.0;
                for (int j = 0; j < h; ++j) {
                    const double dj = variant == 1 ? gelu_tanh_grad(Sp[j]) * dHp[j] : dHp[j];
                    g += dj * Vp[n * h + j];
                }
                const double dal = variant == 1 ? g : g * gelu_tanh_grad(la[tp * L + level]);
                da[tp * L + level] = dal;
                const double *w = W + ((int64_t)p * N + n) * d;
                for (int c = 0; c < d; ++c)
                    dxt[c] += dal * w[c];
            }
        }
    }

    /* Node gradients, one tree per worker, tokens in ascending order. */
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int p = 0; p < P; ++p) {
        double *dWp = dW + (int64_t)p * N * d;
        double *dbp = db + (int64_t)p * N;
        double *dVp = dV + (int64_t)p * N * h;
        for (int64_t i = 0; i < N * d; ++i)
            dWp[i] = 0.0;
        for (int64_t i = 0; i < N; ++i)
            dbp[i] = 0.0;
        for (int64_t i = 0; i < N * h; ++i)
            dVp[i] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tp = t * P + p;
            const double *xt = x + t * d;
            const double *dHp = dH + t * K + (int64_t)p * h;
            const double *Sp = S + t * K + (int64_t)p * h;
            for (int level = 0; level <= D; ++level) {
                const int64_t n = node[tp * L + level];
                const double dal = da[tp * L + level];
                const double a = la[tp * L + level];
                dbp[n] += dal;
                for (int c = 0; c < d; ++c)
                    dWp[n * d + c] += dal * xt[c];
                for (int j = 0; j < h; ++j) {
                    const double cj = variant == 1 ? a * gelu_tanh_grad(Sp[j]) * dHp[j]
                                                   : gelu_tanh(a) * dHp[j];
                    dVp[n * h + j] += cj;
                }
            }
        }
    }

    /* dWout[k,c] = sum_t H[t,k] dy[t,c]. */
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t k = 0; k < K; ++k) {
        double *row = dWout + k * d;
        for (int c = 0; c < d; ++c)
            row[c] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double hk = H[t * K + k];
            const double *dyt = dy + t * d;
            for (int c = 0; c < d; ++c)
                row[c] += hk * dyt[c];
        }
    }
    free(node);
    free(la);
    free(H);
    free(S);
    free(dH);
    free(da);
    free(alive);
    return FFFO_OK;
}
