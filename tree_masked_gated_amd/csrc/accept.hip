// accept.hip -- greedy acceptance walk over each sequence's draft tree, on the
// device, so that the accepted node reaches the commit without a round trip
// through the host (page "Trees from Marginals: Autoregressive drafting with
// factorized priors": the verifier keeps the drafter's guesses that are
// right; section 3: the state is committed once the accepted branch is known).
//
// One wave per sequence.  Lane l holds parent, draft and target token of
// nodes l + 64 k in registers.  Starting from the prefix, each step looks for
// the lowest-index child of the current node whose draft token equals the
// current prediction: a ballot per 64-node chunk, from the chunk holding the
// current node + 1 (children follow their parent), stopping at the first
// chunk with a match.  The walk is as long as the accepted path.
#include <stdint.h>

#include "gdn_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int kAcceptChunks = kMaxNodes / 64;

__global__ __launch_bounds__(64) void accept_kernel(AcceptArgs a) {
    const int b = blockIdx.x, lane = threadIdx.x, N = a.N;
    const int nch = (N + 63) / 64;
    const int32_t* par = a.parent + (size_t)b * N;
    const int32_t* dr = a.draft + (size_t)b * N;
    const int32_t* tg = a.target + (size_t)b * N;
    int pr[kAcceptChunks], dv[kAcceptChunks], tv[kAcceptChunks];
#pragma unroll
    for (int k = 0; k < kAcceptChunks; ++k) {          // unconditional, rows clamped
        const int i = min(lane + 64 * k, N - 1);
        pr[k] = par[i];
        dv[k] = dr[i];
        tv[k] = tg[i];
    }
    int want = a.target_root[b];
    bool bad = false;
#pragma unroll
    for (int k = 0; k < kAcceptChunks; ++k) {
        const int i = lane + 64 * k;
        bad |= __ballot(i < N && (pr[k] < -1 || pr[k] >= i)) != 0ull;
    }
    int cur = -1, len = 0;
    if (bad) {
        len = -1;
    } else {
        for (;;) {
            int found = -1, nwant = 0;
            const int k0 = (cur + 1) >> 6;
#pragma unroll
            for (int k = 0; k < kAcceptChunks; ++k) {
                if (found < 0 && k >= k0 && k < nch) {
                    const int i = lane + 64 * k;
                    const unsigned long long m = __ballot(i < N && pr[k] == cur && dv[k] == want);
                    if (m) {
                        const int l = __ffsll(m) - 1;
                        found = 64 * k + l;
                        nwant = __builtin_amdgcn_readlane(tv[k], l);
                    }
                }
            }
            if (found < 0) break;
            cur = found;
            want = nwant;
            ++len;
        }
    }
    if (lane == 0) {
        a.accepted[b] = cur;
        a.accept_len[b] = len;
        a.next_token[b] = want;
    }
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
    AcceptArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel((const void*)accept_kernel, dim3((unsigned)a.B), dim3(64), args, 0, stream);
}

}  // namespace gdn
