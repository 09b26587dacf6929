// accept.hip -- greedy acceptance walk over each sequence's draft tree, on the
// device, so that the accepted node reaches the commit without a round trip
// through the host (page "Trees from Marginals: Autoregressive drafting with
// factorized priors": the verifier keeps the drafter's guesses that are
// right; section 3: the state is committed once the accepted branch is known).
//
// The walk (from the prefix, to the lowest-index child whose draft token is
// the current prediction, until none is) is evaluated in parallel, one
// workgroup per sequence:
//  1. node i matches if its draft token equals its predecessor's verifier
//     token (the prefix's for a root) and no lower-index sibling matches
//     (an atomic minimum per parent);
//  2. a node is on the walk iff it and all its ancestors match: synchronous
//     pointer doubling carries, per node, the AND of the flags and the size of
//     its covered path segment, log2(depth) + 1 rounds;
//  3. at most one node per depth is on the walk, so the accepted node is the
//     deepest one (a maximum over (depth, index) keys).
#include <stdint.h>

#include "gdn_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int kAcceptThreads = 256;
constexpr int kAcceptPer = kMaxNodes / kAcceptThreads;

__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(AcceptArgs a) {
    __shared__ int32_t s_tg[kMaxNodes];
    __shared__ int32_t s_first[kMaxNodes + 1];    // lowest matching child of parent p, at p + 1
    __shared__ int32_t s_jump[kMaxNodes];
    __shared__ int32_t s_cnt[kMaxNodes];
    __shared__ int32_t s_ok[kMaxNodes];
    __shared__ int s_bad, s_best;
    __shared__ int s_more[3];                     // per-round "a link is left" flags, round r uses r % 3
    const int b = blockIdx.x, tid = threadIdx.x;
    const SeqRows rows = seq_rows(a.offsets, b, a.N);
    const int N = max(rows.n, 0);                   // this tree's nodes
    const int32_t* par = a.parent + rows.row0;
    const int32_t* dr = a.draft + rows.row0;
    const int32_t* tg = a.target + rows.row0;
    const int root = a.target_root[b];
    if (tid == 0) {
        s_bad = 0;
        s_best = -1;
    }
    if (tid < 3) s_more[tid] = 0;
    int p[kAcceptPer], d[kAcceptPer];
#pragma unroll
    for (int k = 0; k < kAcceptPer; ++k) {
        const int i = tid + kAcceptThreads * k;
        p[k] = i < N ? par[i] : -1;
        d[k] = i < N ? dr[i] : 0;
        if (i < N) s_tg[i] = tg[i];
        s_first[i] = 0x7fffffff;
    }
    if (tid == 0) s_first[kMaxNodes] = 0x7fffffff;
    __syncthreads();
    bool bad = false;
#pragma unroll
    for (int k = 0; k < kAcceptPer; ++k) {
        const int i = tid + kAcceptThreads * k;
        bad |= i < N && (p[k] < -1 || p[k] >= i);
    }
    if (bad || rows.n < 0) s_bad = 1;
    __syncthreads();
    const bool invalid = s_bad != 0;
    if (!invalid) {
        bool mt[kAcceptPer];
#pragma unroll
        for (int k = 0; k < kAcceptPer; ++k) {           // 1. matches, lowest per parent
            const int i = tid + kAcceptThreads * k;
            const int pred = p[k] < 0 ? root : s_tg[p[k]];
            mt[k] = i < N && d[k] == pred;
            if (mt[k]) atomicMin(&s_first[p[k] + 1], i);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kAcceptPer; ++k) {
            const int i = tid + kAcceptThreads * k;
            if (i < N) {
                s_ok[i] = mt[k] && s_first[p[k] + 1] == i;
                s_cnt[i] = 1;
                s_jump[i] = p[k];
            }
        }
        __syncthreads();
        // 2. AND over the ancestors.  Round r raises flag r % 3 while some node
        // still has a link to follow and clears flag (r + 1) % 3 before its
        // first barrier (the last readers of that flag finished two rounds
        // earlier): two LDS-only barriers per round, no workgroup reduction.
        for (int rd = 0;; ++rd) {
            int ok[kAcceptPer], cnt[kAcceptPer], nj[kAcceptPer];
            bool more = false;
#pragma unroll
            for (int k = 0; k < kAcceptPer; ++k) {
                const int i = tid + kAcceptThreads * k;
                const int j = i < N ? s_jump[i] : -1;
                ok[k] = 1;
                cnt[k] = 0;
                nj[k] = -1;
                if (j >= 0) {
                    ok[k] = s_ok[j];
                    cnt[k] = s_cnt[j];
                    nj[k] = s_jump[j];
                    more |= nj[k] >= 0;
                }
            }
            if (tid == 0) s_more[(rd + 1) % 3] = 0;
            lds_barrier();
#pragma unroll
            for (int k = 0; k < kAcceptPer; ++k) {
                const int i = tid + kAcceptThreads * k;
                if (i < N && s_jump[i] >= 0) {
                    s_ok[i] &= ok[k];
                    s_cnt[i] += cnt[k];
                    s_jump[i] = nj[k];
                }
            }
            if (more) s_more[rd % 3] = 1;
            lds_barrier();
            if (!s_more[rd % 3]) break;
        }
        int best = -1;                                   // 3. the deepest node on the walk
#pragma unroll
        for (int k = 0; k < kAcceptPer; ++k) {
            const int i = tid + kAcceptThreads * k;
            if (i < N && s_ok[i]) best = max(best, s_cnt[i] * (kMaxNodes + 1) + i);
        }
        if (best >= 0) atomicMax(&s_best, best);
        __syncthreads();
    }
    if (tid == 0) {
        const int key = s_best;
        const int acc = key < 0 ? -1 : key % (kMaxNodes + 1);
        a.accepted[b] = acc;
        a.accept_len[b] = invalid ? -1 : (key < 0 ? 0 : key / (kMaxNodes + 1));
        a.next_token[b] = acc < 0 ? root : s_tg[acc];
    }
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
    AcceptArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel((const void*)accept_kernel, dim3((unsigned)a.B), dim3(kAcceptThreads), args, 0,
                           stream);
}

}  // namespace gdn
