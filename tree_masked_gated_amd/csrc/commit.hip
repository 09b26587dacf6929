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


// d_k = d_v = 128: one workgroup per (sequence, value head).  Each thread owns
// 16 float4 of the 128 x 128 state (rows tid/32 + 8n, columns 4(tid%32)..+3),
// issues all of its S_in loads first, and meanwhile the path is extracted and
// its u and k rows staged in LDS in chunks of kFastChunk nodes.
constexpr int kFastD = 128;
constexpr int kFastChunk = 32;

template <int IO>
__global__ __launch_bounds__(kThreads) void commit_kernel_d128(CommitArgs a) {
    __shared__ __attribute__((aligned(16))) float s_k[kFastChunk * kFastD];
    __shared__ __attribute__((aligned(16))) float s_u[kFastChunk * kFastD];
    __shared__ float s_coef[kFastChunk];
    __shared__ int s_idx[kMaxNodes];

    const int N = a.N, W = (N + 31) / 32;
    const int b = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int tid = threadIdx.x;
    const int r0 = tid >> 5, c4 = (tid & 31) * 4;     // rows r0 + 8n, columns c4..c4+3

    const int acc = a.accepted[b];
    const int status = a.status[b];
    const size_t sbase = ((size_t)b * a.Hv + h) * kFastD * kFastD;
    const float4* Sin = reinterpret_cast<const float4*>(a.S_in + sbase);
    float4* Sout = reinterpret_cast<float4*>(a.S_out + sbase);
    float4 st[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) st[n] = Sin[(r0 + 8 * n) * (kFastD / 4) + (c4 >> 2)];

    const bool valid = status == 0 && acc >= -1 && acc < N;
    const uint32_t* row = a.anc_mask + ((size_t)b * N + (acc < 0 ? 0 : acc)) * W;
    int plen = -1;
    if (valid) plen = acc < 0 ? 0 : row_popc(row, W) + 1;
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
    if (h == 0) {
        int32_t* pb = a.path + (size_t)b * N;
        for (int m = tid; m < N; m += kThreads) pb[m] = m < plen ? s_idx[m] : -1;
        if (tid == 0) a.path_len[b] = plen;
    }
    if (plen <= 0) {                       // nothing accepted (or invalid): S_out = S_in
        if (a.S_in != a.S_out) {
#pragma unroll
            for (int n = 0; n < 16; ++n) Sout[(r0 + 8 * n) * (kFastD / 4) + (c4 >> 2)] = st[n];
        }
        return;
    }
    const float* lg = a.log_gamma + ((size_t)b * a.Hv + h) * N;
    const float* U = a.u + ((size_t)b * a.Hv + h) * (size_t)N * kFastD;
    const float ga = lg[acc];
    const float dec = __expf(ga);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
        st[n].x *= dec; st[n].y *= dec; st[n].z *= dec; st[n].w *= dec;
    }
    for (int p0 = 0; p0 < plen; p0 += kFastChunk) {
        const int pn = min(kFastChunk, plen - p0);
        __syncthreads();
        // stage: 32 threads per node row, 4 consecutive columns each
        for (int x = tid; x < pn * 32; x += kThreads) {
            const int m = x >> 5, c = (x & 31) * 4;
            const int j = s_idx[p0 + m];
            const size_t kb = (((size_t)b * N + j) * a.Hk + hk) * kFastD + c;
            *reinterpret_cast<float4*>(&s_k[m * kFastD + c]) =
                make_float4(ld_io<IO>(a.k, kb), ld_io<IO>(a.k, kb + 1), ld_io<IO>(a.k, kb + 2),
                            ld_io<IO>(a.k, kb + 3));
            *reinterpret_cast<float4*>(&s_u[m * kFastD + c]) =
                *reinterpret_cast<const float4*>(U + (size_t)j * kFastD + c);
        }
        if (tid < pn) s_coef[tid] = __expf(ga - lg[s_idx[p0 + tid]]);
        __syncthreads();
        for (int m = 0; m < pn; ++m) {
            const float4 kv = *reinterpret_cast<const float4*>(&s_k[m * kFastD + c4]);
            const float cm = s_coef[m];
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                const float w = cm * s_u[m * kFastD + r0 + 8 * n];
                st[n].x = fmaf(w, kv.x, st[n].x);
                st[n].y = fmaf(w, kv.y, st[n].y);
                st[n].z = fmaf(w, kv.z, st[n].z);
                st[n].w = fmaf(w, kv.w, st[n].w);
            }
        }
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) Sout[(r0 + 8 * n) * (kFastD / 4) + (c4 >> 2)] = st[n];
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a, int io, hipStream_t stream) {
    CommitArgs copy = a;
    void* args[] = {&copy};
    if (a.dk == kFastD && a.dv == kFastD) {
        const void* fn = io == GDN_BF16 ? (const void*)commit_kernel_d128<GDN_BF16>
                                        : (const void*)commit_kernel_d128<GDN_F32>;
        return hipLaunchKernel(fn, dim3((unsigned)(a.B * a.Hv)), dim3(kThreads), args, 0, stream);
    }
    const void* fn = io == GDN_BF16 ? (const void*)commit_kernel<GDN_BF16>
                                    : (const void*)commit_kernel<GDN_F32>;
    dim3 grid((unsigned)(a.B * a.Hv), (unsigned)((a.dv + kRows - 1) / kRows));
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace gdn
