// commit.hip -- deferred state commit of the accepted draft-tree node.
//
// Page "Trees from Marginals: Autoregressive drafting with factorized priors",
// section 3: the recurrent state is committed only once the accepted branch is
// known, so verification never rolls a state back.  Unrolling the gated delta
// rule along the accepted node a's root-to-node path P gives
//     S_a = e^(G_a) S0 + sum_{j in P} e^(G_a - G_j) u_j k_j^T
// with u_j the rank-one writes and G the path log-gates that verification
// cached; no step of the recurrence is replayed.
//
// Grid: one workgroup per (sequence, value head, block of kRows state rows).
// Each thread owns kRows * d_k / 256 state elements (coalesced along d_k);
// the path's k rows and u values are staged in LDS in chunks of kPathChunk.
// The state stream (S_in read, S_out write) is the dominant HBM traffic.
#include "gdn_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;         // state rows per workgroup
constexpr int kPathChunk = 32;    // path nodes staged per LDS chunk
constexpr int kPerThread = kRows * kMaxHead / kThreads;

template <int IO>
__global__ __launch_bounds__(kThreads) void commit_kernel(CommitArgs a) {
    __shared__ float s_k[kPathChunk * kMaxHead];
    __shared__ float s_u[kPathChunk * kRows];
    __shared__ float s_coef[kPathChunk];
    __shared__ int s_idx[kMaxNodes];

    const int N = a.N, dk = a.dk, dv = a.dv, W = (N + 31) / 32;
    const int unit = blockIdx.x;
    const int b = unit / a.Hv, h = unit % a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int r0 = blockIdx.y * kRows;
    const int nrows = min(kRows, dv - r0);
    const int tid = threadIdx.x;

    const int acc = a.accepted[b];
    const bool valid = a.status[b] == 0 && acc >= -1 && acc < N;
    const uint32_t* row = a.anc_mask + ((size_t)b * N + (acc < 0 ? 0 : acc)) * W;
    int plen = -1;
    if (valid) plen = acc < 0 ? 0 : row_popc(row, W) + 1;

    // path of node acc, root first: its strict ancestors ascending, then acc
    if (plen > 0) {
        for (int w = tid; w < W; w += kThreads) {
            uint32_t x = row[w];
            int base = 0;
            for (int t = 0; t < w; ++t) base += __popc(row[t]);
            while (x) {
                s_idx[base++] = w * 32 + __ffs(x) - 1;
                x &= x - 1u;
            }
        }
        if (tid == 0) s_idx[plen - 1] = acc;
    }
    __syncthreads();
    if (h == 0 && blockIdx.y == 0) {
        int32_t* pb = a.path + (size_t)b * N;
        for (int m = tid; m < N; m += kThreads) pb[m] = m < plen ? s_idx[m] : -1;
        if (tid == 0) a.path_len[b] = plen;
    }

    const size_t sbase = ((size_t)b * a.Hv + h) * (size_t)dv * dk + (size_t)r0 * dk;
    const float* Sin = a.S_in + sbase;
    float* Sout = a.S_out + sbase;
    const int elems = nrows * dk;
    if (plen <= 0) {                       // nothing accepted (or invalid): S_out = S_in
        if (Sin != Sout)
            for (int e = tid; e < elems; e += kThreads) Sout[e] = Sin[e];
        return;
    }

    const float* lg = a.log_gamma + ((size_t)b * a.Hv + h) * N;
    const float* U = a.u + ((size_t)b * a.Hv + h) * (size_t)N * dv;
    const float ga = lg[acc];
    float accv[kPerThread];
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) {
        const int e = tid + t * kThreads;
        accv[t] = e < elems ? __expf(ga) * Sin[e] : 0.f;
    }
    for (int p0 = 0; p0 < plen; p0 += kPathChunk) {
        const int pn = min(kPathChunk, plen - p0);
        __syncthreads();
        for (int x = tid; x < pn * dk; x += kThreads) {
            const int m = x / dk, c = x % dk;
            const int j = s_idx[p0 + m];
            s_k[m * dk + c] = ld_io<IO>(a.k, (((size_t)b * N + j) * a.Hk + hk) * dk + c);
        }
        for (int x = tid; x < pn * nrows; x += kThreads) {
            const int m = x / nrows, r = x % nrows;
            s_u[m * kRows + r] = U[(size_t)s_idx[p0 + m] * dv + r0 + r];
        }
        for (int m = tid; m < pn; m += kThreads) s_coef[m] = __expf(ga - lg[s_idx[p0 + m]]);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kPerThread; ++t) {
            const int e = tid + t * kThreads;
            if (e < elems) {
                const int r = e / dk, c = e % dk;
                float s = accv[t];
                for (int m = 0; m < pn; ++m)
                    s = fmaf(s_coef[m] * s_u[m * kRows + r], s_k[m * dk + c], s);
                accv[t] = s;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) {
        const int e = tid + t * kThreads;
        if (e < elems) Sout[e] = accv[t];
    }
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a, int io, hipStream_t stream) {
    const void* fn = io == GDN_BF16 ? (const void*)commit_kernel<GDN_BF16>
                                    : (const void*)commit_kernel<GDN_F32>;
    CommitArgs copy = a;
    void* args[] = {&copy};
    dim3 grid((unsigned)(a.B * a.Hv), (unsigned)((a.dv + kRows - 1) / kRows));
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace gdn
