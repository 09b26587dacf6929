/*
 * gdn_tree.h -- C ABI of the MI355X (gfx950) library for rollback-free
 * verification of a speculative draft tree through Gated DeltaNet layers.
 *
 * Source of the operation: page "Trees from Marginals: Autoregressive drafting
 * with factorized priors" (gist.science summary of arXiv 2607.06763), section 3
 * "rollback-free tree verification for GDN".  A GDN layer updates its state with
 * the gated delta rule (the state-update equation of that section's "challenge"
 * item).  The section's "solution" items state the method: the tree is
 * topologically sorted, interaction matrices X and Y encode ancestor
 * relations, a linear system (I + X) U = beta V yields every node's output
 * without speculatively updating the recurrent state, and the state is
 * committed only once the accepted branch is known, at the next decoding
 * iteration.  Hence two calls: gdn_tree_verify reads the prefix state and
 * never writes it; gdn_tree_commit writes the accepted node's state.
 *
 * What the calls compute.  Per (sequence b, value head h) unit, with the state
 * S stored d_v x d_k (the page's d_k x d_v state transposed) and value head h
 * reading key head h / (h_v / h_k):
 *
 *     S_i = g_i * S_p(i) * (I - beta_i k_i k_i^T) + beta_i v_i k_i^T,
 *     S_p(i) = S0 when parent[i] = -1,        o_i = S_i q_i,
 *
 * i.e. node i's state is the state reached by running the rule along its own
 * root-to-node path.  The library realises this with the unrolled tree form
 * (Gamma_i = sum of ln g over the path, u_i = S_i - g_i S_p(i) as a rank-one
 * write u_i k_i^T):
 *
 *     (I + X) U = R,  X_ij = beta_i e^(Gamma_i-Gamma_j) k_i.k_j  (j strict ancestor)
 *                     R = diag(beta) (V - diag(e^Gamma) K S0^T)
 *     O = diag(e^Gamma) Q S0^T + Y U,  Y_ij = e^(Gamma_i-Gamma_j) q_i.k_j  (j ancestor or i)
 *     commit:  S_a = e^(Gamma_a) S0 + sum_{j on path(a)} e^(Gamma_a-Gamma_j) u_j k_j^T
 *
 * (the page's right-hand side beta V is the S0 = 0, undecayed special case).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major arrays
 *    owned by the caller, 16-byte aligned.  The library allocates nothing,
 *    never synchronises the device or stream, keeps no global state, and
 *    enqueues its kernels on `stream` (0 = the null stream).  Calls are
 *    asynchronous; every output is valid once the stream reaches them.
 *  - Return value: GDN_OK (0), or a negative gdn_status for an error found on
 *    the host, in which case nothing was launched.  GDN_ERR_LAUNCH means a
 *    kernel launch failed (hipGetLastError after the launch).
 *  - Tree errors are found on the device without a host sync: see
 *    gdn_tree_cache.tree_status.
 *  - The library applies no L2 normalisation and no 1/sqrt(d_k) scale to q or
 *    k; the caller does both.
 *  - batch = 0 is valid and launches nothing.
 *  - Supported sizes: 1 <= n_nodes <= 1024; 1 <= d_k, d_v <= 256; h_k >= 1;
 *    h_v a multiple of h_k.  The fastest kernels cover d_k = d_v = 128.
 */
#ifndef GDN_TREE_H
#define GDN_TREE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o.  bf16 is stored as its 16-bit pattern; the
 * library rounds o to bf16 with round-to-nearest-even. */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,    /* a required pointer is NULL                          */
    GDN_ERR_DIMS = -2,    /* sizes outside the supported range                   */
    GDN_ERR_DTYPE = -3,   /* io_dtype not a gdn_dtype                            */
    GDN_ERR_LAUNCH = -4,  /* a kernel launch failed                              */
    GDN_ERR_ALIGN = -5,   /* a device pointer is not 16-byte aligned             */
    GDN_ERR_ALIAS = -6    /* two caches that must be distinct share a buffer     */
} gdn_status;

/* Problem sizes: B sequences (one draft tree each), N nodes per tree, h_k key
 * heads, h_v value heads, head sizes d_k and d_v, io_dtype a gdn_dtype. */
typedef struct {
    int32_t batch, n_nodes, h_k, h_v, d_k, d_v, io_dtype;
} gdn_tree_dims;

/* Per-call state written by gdn_tree_verify and read by gdn_tree_commit.
 * Caller-allocated device buffers, sizes from gdn_tree_cache_bytes. */
typedef struct {
    /* [B][N][ceil(N/32)]: bit (j % 32) of word j / 32 of row i is set iff node
     * j is a strict ancestor of node i; padding bits are zero.  Rows of an
     * invalid tree are zero. */
    uint32_t* anc_mask;
    /* [B][N]: number of strict ancestors of each node (depth; 0 under S0),
     * -1 for every node of an invalid tree. */
    int32_t* depth;
    /* [B][H_v][N][d_v] fp32: the rank-one write u_i of every node. */
    float* u;
    /* [B][H_v][N] fp32: Gamma_i, the sum of ln g over node i's path. */
    float* log_gamma;
    /* [B]: 0 when the tree is valid, else i + 1 for the first node i whose
     * parent is outside [-1, i).  The o rows of an invalid tree are NaN. */
    int32_t* tree_status;
} gdn_tree_cache;

/* Byte sizes of the five cache buffers for `dims` (any pointer may be NULL to
 * skip it).  Returns GDN_OK, GDN_ERR_NULL (dims NULL) or the size errors of
 * gdn_tree_verify. */
int gdn_tree_cache_bytes(const gdn_tree_dims* dims, size_t* anc_mask, size_t* depth,
                         size_t* u, size_t* log_gamma, size_t* tree_status);

/*
 * Verify every node of every tree in one pass (section 3, the masked triangular
 * solve and the single-pass output stage).
 *
 *   S0      [B][H_v][d_v][d_k] fp32    prefix state; read only, never written
 *   q, k    [B][N][H_k][d_k]   io      queries and keys per key head
 *   v       [B][N][H_v][d_v]   io      values per value head
 *   beta, g [B][N][H_v]        fp32    write strength and gate, g in (0, 1]
 *   parent  [B][N]             int32   -1 = follows S0, else an index < i
 *   o       [B][N][H_v][d_v]   io      out: o_i = S_i q_i
 *   cache                               out: see gdn_tree_cache
 *
 * The tree must list parents before children (a topological order); the
 * library validates this on the device and does not reorder nodes.
 */
int gdn_tree_verify(const gdn_tree_dims* dims, const float* S0, const void* q,
                    const void* k, const void* v, const float* beta, const float* g,
                    const int32_t* parent, void* o, const gdn_tree_cache* cache,
                    hipStream_t stream);

/*
 * Commit the accepted node's state (section 3, deferred state commitment):
 * S_out = S_a for a = accepted[b], from the cached u and Gamma, without
 * replaying the recurrence.
 *
 *   S_in     [B][H_v][d_v][d_k] fp32  the S0 that gdn_tree_verify read
 *   S_out    [B][H_v][d_v][d_k] fp32  out; may alias S_in (in-place commit)
 *   k        [B][N][H_k][d_k]   io    the keys given to gdn_tree_verify
 *   cache                              as written by gdn_tree_verify
 *   accepted [B]                int32 accepted node, or -1 for none
 *   path     [B][N]             int32 out: root..accepted, -1 padded
 *   path_len [B]                int32 out: path length; 0 when accepted = -1;
 *                                     -1 when the tree is invalid or accepted
 *                                     is outside [-1, N) -- then S_out = S_in
 *
 * k and the cache must be unchanged since gdn_tree_verify, with the same dims.
 */
int gdn_tree_commit(const gdn_tree_dims* dims, const float* S_in, float* S_out,
                    const void* k, const gdn_tree_cache* cache, const int32_t* accepted,
                    int32_t* path, int32_t* path_len, hipStream_t stream);

/*
 * One decode step with the commit deferred into it (section 3: the state is
 * committed once the accepted branch is known, and the pages' design folds it
 * into the next iteration).  The results are those of
 *
 *   gdn_tree_commit(dims, S_prev, S_new, k_prev, cache_prev, accepted_prev,
 *                   path_prev, path_len_prev, stream);
 *   gdn_tree_verify(dims, S_new, q, k, v, beta, g, parent, o, cache, stream);
 *
 * but S_prev is read once: the committed state is formed on chip, written to
 * S_new and used directly as the new tree's prefix state (fp32 rounding order
 * may differ from the two-call sequence).
 *
 *   S_prev, S_new  [B][H_v][d_v][d_k] fp32  S_new may alias S_prev
 *   k_prev, cache_prev, accepted_prev, path_prev, path_len_prev
 *                  as for gdn_tree_commit (the previous tree)
 *   q, k, v, beta, g, parent, o, cache
 *                  as for gdn_tree_verify (the new tree)
 *
 * Both trees have the shape dims.  cache_prev is read while cache is written,
 * so no buffer of one may be a buffer of the other (GDN_ERR_ALIAS); a decode
 * loop alternates two caches.  Every size gdn_tree_verify accepts is
 * accepted; the single-pass form covers d_k = d_v = 128 with bf16 io and
 * N <= 128, other sizes run the two calls.
 */
int gdn_tree_commit_verify(const gdn_tree_dims* dims, const float* S_prev, float* S_new,
                           const void* k_prev, const gdn_tree_cache* cache_prev,
                           const int32_t* accepted_prev, int32_t* path_prev,
                           int32_t* path_len_prev, const void* q, const void* k,
                           const void* v, const float* beta, const float* g,
                           const int32_t* parent, void* o, const gdn_tree_cache* cache,
                           hipStream_t stream);

/*
 * Greedy acceptance walk over each sequence's draft tree, on the device (page
 * "Trees from Marginals", the speculative-decoding item: the verifier keeps
 * the drafter's guesses that are right; section 3: the state is committed
 * once the accepted branch is known).  With it, the accepted node reaches
 * gdn_tree_commit / gdn_tree_commit_verify without a host round trip.
 *
 *   parent      [B][N] int32  the tree, as for gdn_tree_verify
 *   draft       [B][N] int32  each node's draft token
 *   target      [B][N] int32  the verifier's token after each node (argmax of
 *                             its logits at that node)
 *   target_root [B]    int32  the verifier's token after the prefix
 *   accepted    [B]    int32  out: the accepted node, -1 if none
 *   accept_len  [B]    int32  out: nodes accepted (depth + 1), 0 if none,
 *                             -1 for an invalid parent row
 *   next_token  [B]    int32  out: the verifier's token after the accepted
 *                             tokens (target_root if none)
 *
 * From the prefix, the walk moves to the lowest-index child whose draft token
 * equals the current prediction and stops where no child matches.  Only
 * dims->batch and dims->n_nodes are used (the other fields are checked as for
 * the other calls).  An invalid parent row gives accepted = -1.
 */
int gdn_tree_accept(const gdn_tree_dims* dims, const int32_t* parent, const int32_t* draft,
                    const int32_t* target, const int32_t* target_root, int32_t* accepted,
                    int32_t* accept_len, int32_t* next_token, hipStream_t stream);

/*
 * Ragged batches.  The trees of one batch may differ in size: the pages run
 * draft budgets of 16 and 64 nodes (page "Technisches Resuemee: TreeFlash",
 * experimental results) and leave batches of several sequences open (its
 * limitations item), so a batch that mixes budgets is the serving case.  The
 * *_ragged calls take the per-node arrays packed, sequence after sequence:
 *
 *   offsets [B + 1] int32, DEVICE: sequence b owns rows offsets[b] ..
 *           offsets[b+1] - 1 of every per-node array, n_b = offsets[b+1] -
 *           offsets[b] nodes (0 allowed), offsets[0] = 0, non-decreasing;
 *           T = offsets[B] rows in all.  4-byte aligned (else GDN_ERR_ALIGN),
 *           not NULL (else GDN_ERR_NULL).
 *   dims->n_nodes = N, the largest tree allowed (every n_b <= N): the cache
 *           keeps its [B][N] layout and sizes (gdn_tree_cache_bytes), the
 *           kernels are chosen by N, and a tree of n_b < N nodes computes
 *           only its own rows.
 *
 * Per-node arrays become [T][...]: q, k [T][H_k][d_k]; v, o [T][H_v][d_v];
 * beta, g [T][H_v]; parent, draft, target, and a commit's path [T] (indices
 * local to their tree: parent -1 or < i; path holds root..accepted, then -1,
 * in the tree's own n_b slots).  Cache rows i >= n_b: anc_mask zero, depth
 * -1, u and log_gamma unspecified.  The offsets are read on the device: a
 * sequence with offsets[b] < 0 or n_b outside [0, N] gets tree_status -1,
 * none of its rows is read or written, its commit gives path_len -1 and
 * S_out = S_in, and its acceptance accepted = -1, accept_len = -1.  The
 * caller guarantees that every array holds T rows.  An empty tree (n_b = 0)
 * is valid: nothing to verify, and only accepted = -1 commits it.
 * Otherwise each call behaves as its dense form on each tree alone.
 */
int gdn_tree_verify_ragged(const gdn_tree_dims* dims, const int32_t* offsets, const float* S0,
                           const void* q, const void* k, const void* v, const float* beta,
                           const float* g, const int32_t* parent, void* o,
                           const gdn_tree_cache* cache, hipStream_t stream);

/* offsets: the verified tree's, as given to gdn_tree_verify_ragged. */
int gdn_tree_commit_ragged(const gdn_tree_dims* dims, const int32_t* offsets, const float* S_in,
                           float* S_out, const void* k, const gdn_tree_cache* cache,
                           const int32_t* accepted, int32_t* path, int32_t* path_len,
                           hipStream_t stream);

/* offsets_prev: the previous tree's (k_prev, path_prev); offsets: the new
 * tree's (q, k, v, beta, g, parent, o).  Both trees have at most N nodes. */
int gdn_tree_commit_verify_ragged(const gdn_tree_dims* dims, const int32_t* offsets_prev,
                                  const float* S_prev, float* S_new, const void* k_prev,
                                  const gdn_tree_cache* cache_prev, const int32_t* accepted_prev,
                                  int32_t* path_prev, int32_t* path_len_prev,
                                  const int32_t* offsets, const void* q, const void* k,
                                  const void* v, const float* beta, const float* g,
                                  const int32_t* parent, void* o, const gdn_tree_cache* cache,
                                  hipStream_t stream);

int gdn_tree_accept_ragged(const gdn_tree_dims* dims, const int32_t* offsets, const int32_t* parent,
                           const int32_t* draft, const int32_t* target, const int32_t* target_root,
                           int32_t* accepted, int32_t* accept_len, int32_t* next_token,
                           hipStream_t stream);

/*
 * Draft-tree construction with w expansions per step (page "Trees from
 * Marginals", section 2, tree construction: best-first expansion as in
 * DySpec, changed so that the w best candidates leave the candidate heap
 * together and are expanded together, building a tree of N nodes in
 * ceil(N / w) sequential steps).  The drafter itself is outside this library:
 * its outputs are the input.
 *
 *   logp [B][N + 1][K] fp32   row 0: log-probabilities of the drafter's K
 *                             continuations of the prefix; row 1 + i: those
 *                             of node i (the node that receives index i)
 *   tok  [B][N + 1][K] int32  the continuations' tokens, same layout
 *   parent [B][N] int32  out: the tree, topologically ordered (parent[i] < i,
 *                             -1 under the prefix): gdn_tree_verify's input
 *   token  [B][N] int32  out: each node's token (its draft token for
 *                             gdn_tree_accept)
 *   score  [B][N] fp32   out: each node's score
 *
 * A candidate is the continuation of rank c after a node p already in the
 * tree (p = -1: the prefix); its score is score(p) + logp[p + 1][c], one fp32
 * addition, with score(prefix) = 0.  Each step takes the min(w, N - n, open
 * candidates) best ones, ordered by score (higher first), then p, then c
 * (lower first), makes them nodes n, n + 1, ... in that order, and opens the
 * K continuations of each.  logp must hold no NaN.
 *
 * Sizes: 1 <= N <= 1024, 1 <= K <= 64, w >= 1, and the per-sequence working
 * set, about 8 (2N + pow2(min(w, N) K)) + 4 (N + 1) K + 12 N bytes, within the
 * 160 KiB of LDS (else GDN_ERR_DIMS).  batch = 0 launches nothing.
 */
typedef struct {
    int32_t batch, n_nodes, topk, width;
} gdn_tree_build_dims;

int gdn_tree_build(const gdn_tree_build_dims* dims, const float* logp, const int32_t* tok,
                   int32_t* parent, int32_t* token, float* score, hipStream_t stream);

/* Static description of a gdn_status value. */
const char* gdn_tree_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_TREE_H */
