/*
 * gdn_oracle.c -- plain, slow, fp64 CPU oracle for draft-tree verification
 * through Gated DeltaNet (GDN) layers.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP library; the two meet only in the seeded input
 * generator, which holds none of the method's arithmetic.
 *
 * What it computes (page "Trees from Marginals: Autoregressive drafting with
 * factorized priors", section 3 "rollback-free tree verification for GDN",
 * state-update equation of the "challenge" item): every tree node's state is
 * the state reached by running the gated delta rule sequentially along that
 * node's own root-to-node path, starting from the prefix state S0.  We store S
 * as d_v x d_k (row r = value coordinate, column c = key coordinate); the
 * page's d_k x d_v form  S_t = a_t (I - b_t k k^T) S_{t-1} + b_t k v^T  is its
 * exact transpose, with a_t the gate g:
 *
 *     S <- g * S * (I - beta k k^T) + beta v k^T ,     o_i = S_i q_i .
 *
 * The decay multiplies the whole transition but not the new write, and the
 * output of node i is read from the state after node i's own update.
 *
 * Tree conventions (same section, "the tree is topologically sorted" item):
 * parent[i] = -1 means node i follows the prefix state S0 directly, otherwise
 * parent[i] must lie in [0, i).  The first node violating this makes the whole
 * tree invalid: status = i + 1, outputs NaN, nothing committed.
 *
 * Deferred commit (same section, "state commitment is deferred" item): the
 * state to commit is the state of the accepted node, or S0 when the accepted
 * index is -1 (nothing accepted); path lists the accepted node's root-to-node
 * path, root first.  An accepted index outside [-1, N) gives path_len = -1 and
 * S0 as the committed state.
 *
 * Auxiliary outputs, also straight from the recurrence:
 *   u_i = beta_i (v_i - g_i S_{parent(i)} k_i)   the rank-one write of node i's
 *         step, i.e. S_i = g_i S_{parent(i)} + u_i k_i^T;
 *   log_gamma_i = sum of ln g_j over node i's root-to-node path (inclusive).
 *
 * Evaluation order is fixed: w = S k with the sum over c ascending, then
 * S[r][c] = g * (S[r][c] - beta * w[r] * k[c]) + beta * v[r] * k[c].
 * Build with -ffp-contract=off so every machine rounds the same way.
 *
 * Two modes give bit-identical results: mode 0 walks each node's whole path
 * from S0; mode 1 (memo) applies the same single step to the stored parent
 * state, which is the same sequence of fp64 operations.
 *
 * Parity pins: the single step against a gradient step of the online
 * regression loss (autograd), closed forms (beta = 0 pure decay; beta = 1 with
 * q = k of unit norm returns v), a chain against the product form of the
 * linear recurrence, ancestor masks against a boolean transitive closure,
 * whole trees against a dense linear solve, and tree invariants (siblings,
 * non-ancestors, relabelling).  See the tests that load this library.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ trees */

/* Validate one tree and return 0, or i+1 for the first node with a bad parent. */
static int tree_check(int n, const int32_t* par)
{
    for (int i = 0; i < n; ++i)
        if (par[i] < -1 || par[i] >= i) return i + 1;
    return 0;
}

/* Root-to-node path of node i (root first) into out; returns its length. */
static int tree_path(const int32_t* par, int i, int32_t* out)
{
    int len = 0;
    for (int j = i; j >= 0; j = par[j]) out[len++] = j;
    for (int a = 0, b = len - 1; a < b; ++a, --b) {
        int32_t t = out[a]; out[a] = out[b]; out[b] = t;
    }
    return len;
}

/*
 * Per sequence b: status[b], depth[b][i] (= path length - 1, so a node under
 * the prefix has depth 0) and strict-ancestor bit rows
 * mask[b][i][w] (bit j%32 of word j/32 set <=> j is a strict ancestor of i;
 * unused high bits zero).  Rows of an invalid tree are left zero, depth -1.
 */
int oracle_tree(int B, int N, const int32_t* parent, uint32_t* mask,
                int32_t* depth, int32_t* status)
{
    if (B < 0 || N < 1) return -1;
    const int W = (N + 31) / 32;
    int32_t* path = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    if (!path) return -2;
    for (int b = 0; b < B; ++b) {
        const int32_t* par = parent + (size_t)b * N;
        uint32_t* mb = mask + (size_t)b * N * W;
        memset(mb, 0, sizeof(uint32_t) * (size_t)N * W);
        status[b] = tree_check(N, par);
        for (int i = 0; i < N; ++i) {
            if (status[b]) { depth[(size_t)b * N + i] = -1; continue; }
            int len = tree_path(par, i, path);
            depth[(size_t)b * N + i] = len - 1;
            for (int m = 0; m + 1 < len; ++m)
                mb[(size_t)i * W + path[m] / 32] |= 1u << (path[m] % 32);
        }
    }
    free(path);
    return 0;
}

/* ------------------------------------------------------------ recurrence */

/*
 * Greedy acceptance walk over one tree per sequence (page "Trees from
 * Marginals", the speculative-decoding item: the drafter guesses, the verifier
 * checks the guesses and keeps the ones that are right; section 3: the state
 * is committed once the accepted branch is known).  Reading taken: greedy
 * verification of a token tree.  target_root[b] is the verifier's token after
 * the prefix and target[b][i] its token after node i (the argmax of its
 * logits at that position).  Starting at the prefix, the walk moves to the
 * first child (lowest index) whose draft token equals the current prediction,
 * and stops when no child matches:
 *     accepted[b]   = the last node reached, -1 if no root node matched;
 *     accept_len[b] = the number of nodes reached (its depth + 1, or 0);
 *     next_token[b] = the prediction at that point (the verifier's token that
 *                     follows the accepted tokens).
 * An invalid parent row gives accepted = -1, accept_len = -1 and
 * next_token = target_root[b].
 */
int oracle_accept(int B, int N, const int32_t* parent, const int32_t* draft,
                  const int32_t* target, const int32_t* target_root, int32_t* accepted,
                  int32_t* accept_len, int32_t* next_token)
{
    if (B < 0 || N < 1) return -1;
    for (int b = 0; b < B; ++b) {
        const int32_t* par = parent + (size_t)b * N;
        const int32_t* dr = draft + (size_t)b * N;
        const int32_t* tg = target + (size_t)b * N;
        int want = target_root[b];
        if (tree_check(N, par)) {
            accepted[b] = -1;
            accept_len[b] = -1;
            next_token[b] = want;
            continue;
        }
        int cur = -1, len = 0;
        for (;;) {
            int found = -1;
            for (int i = 0; i < N; ++i)
                if (par[i] == cur && dr[i] == want) {
                    found = i;
                    break;
                }
            if (found < 0) break;
            cur = found;
            want = tg[cur];
            ++len;
        }
        accepted[b] = cur;
        accept_len[b] = len;
        next_token[b] = want;
    }
    return 0;
}

/*
 * Draft-tree construction with w expansions per step (the pages' section 2,
 * "tree construction": DySpec's best-first expansion, changed so that the w
 * best candidates leave the candidate heap together and are expanded
 * together, which builds a tree of N nodes in ceil(N / w) sequential steps).
 * The drafter is replaced by synthetic scores given as input:
 *   logp[b][r][c], tok[b][r][c], r = 0 .. N, c < K: row 0 holds the drafter's
 *   K continuations of the prefix (log-probability, token), row 1 + i those of
 *   node i (whatever node receives index i).
 * A candidate is the continuation of rank c after a node p (p = -1: the
 * prefix); its score is score(p) + logp[b][p + 1][c], with score(prefix) = 0,
 * one fp32 addition (so the selections are decided in fp32, as the kernel
 * decides them).  Candidates are ordered by score, higher first, then by p,
 * then by c, lower first.  Each step takes the first m = min(w, N - n, number
 * of candidates) of them, makes them nodes n, n + 1, ... in that order
 * (parent p, token tok[b][p + 1][c], that score), removes them, and adds the K
 * children of each.  Steps repeat until the tree has N nodes.
 * Returns 0, or -1 for bad sizes, -2 when out of memory.
 */
typedef struct {
    float s;
    int32_t p, c;
} cand_t;

static int cand_cmp(const void* x, const void* y)
{
    const cand_t* a = (const cand_t*)x;
    const cand_t* b = (const cand_t*)y;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    if (a->p != b->p) return a->p < b->p ? -1 : 1;
    return a->c < b->c ? -1 : (a->c > b->c);
}

int oracle_build(int B, int N, int K, int w, const float* logp, const int32_t* tok,
                 int32_t* parent, int32_t* token, float* score)
{
    if (B < 0 || N < 1 || K < 1 || w < 1) return -1;
    cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)K * (N + 1));
    if (!cand) return -2;
    for (int b = 0; b < B; ++b) {
        const float* lp = logp + (size_t)b * (N + 1) * K;
        const int32_t* tk = tok + (size_t)b * (N + 1) * K;
        int32_t* par = parent + (size_t)b * N;
        int32_t* out_tok = token + (size_t)b * N;
        float* sc = score + (size_t)b * N;
        int nc = 0, n = 0;
        for (int c = 0; c < K; ++c) {
            cand[nc].s = 0.0f + lp[c];
            cand[nc].p = -1;
            cand[nc].c = c;
            ++nc;
        }
        while (n < N) {
            qsort(cand, (size_t)nc, sizeof(cand_t), cand_cmp);
            int m = w;
            if (m > N - n) m = N - n;
            if (m > nc) m = nc;
            const int first = n;
            for (int t = 0; t < m; ++t, ++n) {
                par[n] = cand[t].p;
                out_tok[n] = tk[(size_t)(cand[t].p + 1) * K + cand[t].c];
                sc[n] = cand[t].s;
            }
            memmove(cand, cand + m, sizeof(cand_t) * (size_t)(nc - m));
            nc -= m;
            for (int i = first; i < n; ++i)
                for (int c = 0; c < K; ++c) {
                    cand[nc].s = sc[i] + lp[(size_t)(i + 1) * K + c];
                    cand[nc].p = i;
                    cand[nc].c = c;
                    ++nc;
                }
        }
    }
    free(cand);
    return 0;
}

/* One gated delta step on S (dv x dk, row-major), in the fixed order above. */
static void gdn_step(int dv, int dk, double* S, const double* k, const double* v,
                     double beta, double g, double* w)
{
    for (int r = 0; r < dv; ++r) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += S[(size_t)r * dk + c] * k[c];
        w[r] = acc;
    }
    for (int r = 0; r < dv; ++r) {
        for (int c = 0; c < dk; ++c) {
            double s = S[(size_t)r * dk + c];
            S[(size_t)r * dk + c] = g * (s - beta * w[r] * k[c]) + beta * v[r] * k[c];
        }
    }
}

/* o = S q, sum over c ascending. */
static void state_times(int dv, int dk, const double* S, const double* q, double* o)
{
    for (int r = 0; r < dv; ++r) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += S[(size_t)r * dk + c] * q[c];
        o[r] = acc;
    }
}

typedef struct {
    int B, N, Hk, Hv, dk, dv;
    const double *S0, *q, *k, *v, *beta, *g;
    const int32_t *parent, *accepted;
} problem;

/* index helpers for the documented layouts */
static size_t ix_qk(const problem* P, int b, int i, int h) /* [B][N][Hk][dk] */
{ return (((size_t)b * P->N + i) * P->Hk + h) * P->dk; }
static size_t ix_v(const problem* P, int b, int i, int h)  /* [B][N][Hv][dv] */
{ return (((size_t)b * P->N + i) * P->Hv + h) * P->dv; }
static size_t ix_bg(const problem* P, int b, int i, int h) /* [B][N][Hv] */
{ return ((size_t)b * P->N + i) * P->Hv + h; }
static size_t ix_S(const problem* P, int b, int h)          /* [B][Hv][dv][dk] */
{ return ((size_t)b * P->Hv + h) * (size_t)P->dv * P->dk; }
static size_t ix_u(const problem* P, int b, int h, int i)   /* [B][Hv][N][dv] */
{ return (((size_t)b * P->Hv + h) * P->N + i) * P->dv; }

/*
 * One (sequence b, value head h) unit.  Value head h reads key head
 * h / (Hv / Hk).  Writes o, u, log_gamma and the committed state.
 */
static void run_unit(const problem* P, int b, int h, int memo, int status,
                     double* o, double* u, double* lg, double* S_commit)
{
    const int N = P->N, dv = P->dv, dk = P->dk;
    const int hk = h / (P->Hv / P->Hk);
    const size_t SS = (size_t)dv * dk;
    const int32_t* par = P->parent + (size_t)b * N;
    const double* S0 = P->S0 + ix_S(P, b, h);
    const int acc = P->accepted[b];
    double* Sc = S_commit + ix_S(P, b, h);

    memcpy(Sc, S0, sizeof(double) * SS);   /* default commit: nothing accepted */
    if (status) {
        for (int i = 0; i < N; ++i) {
            for (int r = 0; r < dv; ++r) o[ix_v(P, b, i, h) + r] = NAN;
            for (int r = 0; r < dv; ++r) u[ix_u(P, b, h, i) + r] = NAN;
            lg[((size_t)b * P->Hv + h) * N + i] = NAN;
        }
        return;
    }

    double* w = (double*)malloc(sizeof(double) * (size_t)dv);
    int32_t* path = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    /* memo keeps every node's state; the path walk keeps one working state */
    double* S = (double*)malloc(sizeof(double) * SS * (memo ? (size_t)N : 1));

    for (int i = 0; i < N; ++i) {
        double* Si = memo ? S + (size_t)i * SS : S;
        const double* kb = P->k + ix_qk(P, b, i, hk);
        const double* vb = P->v + ix_v(P, b, i, h);
        const double bi = P->beta[ix_bg(P, b, i, h)];
        const double gi = P->g[ix_bg(P, b, i, h)];
        double lgi;
        if (memo) {
            const double* Sp = par[i] < 0 ? S0 : S + (size_t)par[i] * SS;
            memcpy(Si, Sp, sizeof(double) * SS);
            lgi = (par[i] < 0 ? 0.0 : lg[((size_t)b * P->Hv + h) * N + par[i]]) + log(gi);
        } else {
            int len = tree_path(par, i, path);
            memcpy(Si, S0, sizeof(double) * SS);
            lgi = 0.0;
            for (int m = 0; m + 1 < len; ++m) {
                int j = path[m];
                gdn_step(dv, dk, Si, P->k + ix_qk(P, b, j, hk), P->v + ix_v(P, b, j, h),
                         P->beta[ix_bg(P, b, j, h)], P->g[ix_bg(P, b, j, h)], w);
                lgi += log(P->g[ix_bg(P, b, j, h)]);
            }
            lgi += log(gi);
        }
        /* Si now holds the parent's state: record the write vector u_i. */
        state_times(dv, dk, Si, kb, w);
        for (int r = 0; r < dv; ++r)
            u[ix_u(P, b, h, i) + r] = bi * (vb[r] - gi * w[r]);
        gdn_step(dv, dk, Si, kb, vb, bi, gi, w);
        lg[((size_t)b * P->Hv + h) * N + i] = lgi;
        state_times(dv, dk, Si, P->q + ix_qk(P, b, i, hk), o + ix_v(P, b, i, h));
        if (i == acc) memcpy(Sc, Si, sizeof(double) * SS);
    }
    free(S);
    free(path);
    free(w);
}

/*
 * Verify every node of every tree and produce the state to commit.
 *
 * Inputs (float64, the exact values the GPU library reads, widened):
 *   S0 [B][Hv][dv][dk], q, k [B][N][Hk][dk], v [B][N][Hv][dv],
 *   beta, g [B][N][Hv], parent [B][N], accepted [B].
 * Outputs: o [B][N][Hv][dv], u [B][Hv][N][dv], log_gamma [B][Hv][N],
 *   S_commit [B][Hv][dv][dk], path [B][N] (root first, -1 padded),
 *   path_len [B], status [B].
 * memo: 0 = walk every path from S0, 1 = reuse the parent's stored state.
 * nthreads: OpenMP threads over (b, h) units, 0 = runtime default.
 * Returns 0, or a negative value for bad sizes / allocation failure.
 */
int oracle_verify(int B, int N, int Hk, int Hv, int dk, int dv,
                  const double* S0, const double* q, const double* k,
                  const double* v, const double* beta, const double* g,
                  const int32_t* parent, const int32_t* accepted, int memo,
                  int nthreads, double* o, double* u, double* log_gamma,
                  double* S_commit, int32_t* path, int32_t* path_len,
                  int32_t* status)
{
    if (B < 0 || N < 1 || Hk < 1 || Hv < 1 || Hv % Hk || dk < 1 || dv < 1) return -1;
    problem P = {B, N, Hk, Hv, dk, dv, S0, q, k, v, beta, g, parent, accepted};

    for (int b = 0; b < B; ++b) {
        const int32_t* par = parent + (size_t)b * N;
        int32_t* pb = path + (size_t)b * N;
        for (int i = 0; i < N; ++i) pb[i] = -1;
        status[b] = tree_check(N, par);
        const int a = accepted[b];
        if (status[b] || a < -1 || a >= N) path_len[b] = -1;
        else if (a == -1) path_len[b] = 0;
        else path_len[b] = tree_path(par, a, pb);
    }

    const long units = (long)B * Hv;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (long t = 0; t < units; ++t) {
        int b = (int)(t / Hv), h = (int)(t % Hv);
        run_unit(&P, b, h, memo, status[b], o, u, log_gamma, S_commit);
    }
    /* an accepted index outside [-1, N) matches no node: run_unit left S0 */
    return 0;
}

/* Threads the OpenMP runtime would use (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
