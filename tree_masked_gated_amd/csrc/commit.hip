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
    const SeqRows rows = seq_rows(a.offsets, b, N);
    const bool valid = a.status[b] == 0 && rows.n >= 0 && acc >= -1 && acc < rows.n;
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
        int32_t* pb = a.path + rows.row0;
        for (int m = tid; m < rows.n; m += kThreads) pb[m] = m < plen ? s_idx[m] : -1;
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
            s_k[m * dk + c] = ld_io<IO>(a.k, ((rows.row0 + j) * a.Hk + hk) * dk + c);
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

    const SeqRows rows = seq_rows(a.offsets, b, N);
    const bool valid = status == 0 && rows.n >= 0 && acc >= -1 && acc < rows.n;
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
        int32_t* pb = a.path + rows.row0;
        for (int m = tid; m < rows.n; m += kThreads) pb[m] = m < plen ? s_idx[m] : -1;
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
            const size_t kb = ((rows.row0 + j) * a.Hk + hk) * kFastD + c;
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


// d_k = d_v = 128 with bf16 k: the path's rank-one updates as one product on
// the 16x16x32 MFMA.  With w_j = e^(G_a - G_j) and D = S^T (rows: key column
// c, columns: value row r),
//     D_out = e^(G_a) D_in + K_P^T (diag(w) U_P),
// K_P (|P| x 128) the path's k rows and U_P (|P| x 128, fp32) its u rows.
// Two workgroups per (sequence, value head), one per half of the value rows
// (the update of a row needs only that row's u entries); four waves, wave w
// owns value-row tile w of its half and all eight key-column tiles: 8
// accumulator tiles whose lanes hold 4 consecutive key columns of one value
// row, i.e. 16 contiguous bytes of S, so S_in loads and S_out stores stay
// row-major.  The path is consumed 64 nodes at a time (a chunk's loads are
// one HBM round trip, so fewer, larger chunks): its k rows and its weighted
// u rows (split into bf16 hi + lo, about 16 mantissa bits, so the update
// keeps fp32-level accuracy) are staged transposed in LDS, each MFMA operand
// one 16-byte read, the next chunk's loads issued before the current chunk's
// products.
constexpr int kMfmaChunk = 64;
constexpr int kMfmaHalves = 2;                       // value-row halves per (b, h)
constexpr int kHalfRows = kFastD / kMfmaHalves;

__global__ __launch_bounds__(kThreads) void commit_kernel_mfma(CommitArgs a) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) uint16_t s_kT[kFastD * kMfmaChunk];      // [c][j]
    __shared__ __attribute__((aligned(16))) uint16_t s_uhT[kHalfRows * kMfmaChunk];  // [r][j], hi
    __shared__ __attribute__((aligned(16))) uint16_t s_ulT[kHalfRows * kMfmaChunk];  // [r][j], lo
    __shared__ int s_idx[kMaxNodes];

    const int N = a.N, W = (N + 31) / 32;
    const int half = blockIdx.x % kMfmaHalves, bh = blockIdx.x / kMfmaHalves;
    const int b = bh / a.Hv, h = bh % a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lq = lane >> 4, wave = tid >> 6;
    const int r0 = half * kHalfRows;                  // this workgroup's first value row

    const int acc_node = a.accepted[b];
    const int status = a.status[b];
    const size_t sbase = ((size_t)b * a.Hv + h) * kFastD * kFastD;
    const size_t srow = sbase + (size_t)(r0 + 16 * wave + ln) * kFastD + 4 * lq;
    f32x4 D[8];                                       // [key-column tile], value-row tile `wave`
#pragma unroll
    for (int tc = 0; tc < 8; ++tc) D[tc] = *reinterpret_cast<const f32x4*>(a.S_in + srow + 16 * tc);

    const SeqRows rows = seq_rows(a.offsets, b, N);
    const bool valid = status == 0 && rows.n >= 0 && acc_node >= -1 && acc_node < rows.n;
    const uint32_t* row = a.anc_mask + ((size_t)b * N + (acc_node < 0 ? 0 : acc_node)) * W;
    int plen = -1;
    if (valid) plen = acc_node < 0 ? 0 : row_popc(row, W) + 1;
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
        if (tid == 0) s_idx[plen - 1] = acc_node;
    }
    __syncthreads();
    if (h == 0 && half == 0) {
        int32_t* pb = a.path + rows.row0;
        for (int m = tid; m < rows.n; m += kThreads) pb[m] = m < plen ? s_idx[m] : -1;
        if (tid == 0) a.path_len[b] = plen;
    }
    if (plen > 0) {
        const float* lg = a.log_gamma + ((size_t)b * a.Hv + h) * N;
        const float* U = a.u + ((size_t)b * a.Hv + h) * (size_t)N * kFastD;
        const uint16_t* K = static_cast<const uint16_t*>(a.k);
        const float ga = lg[acc_node];
        const float dec = __expf(ga);
#pragma unroll
        for (int tc = 0; tc < 8; ++tc) D[tc] *= dec;
        // staging: path node m of the chunk, key columns kseg .. +31 and value
        // rows useg .. +15 of this half.  The lanes of a wave take the chunk's
        // 64 nodes in order, so each transposed 2-byte store of a wave fills
        // one 128-byte row of the staging tile (no two lanes in one bank but
        // the two halves of a 4-byte word).
        const int m = tid & 63, kseg = (tid >> 6) * 32, useg = (tid >> 6) * 16;
        static_assert(kThreads == 64 * 4 && kMfmaChunk == 64 && kHalfRows == 4 * 16,
                      "64 nodes x 4 column segments");
        // chunk loads, unconditional (rows past the path re-read its last node
        // with weight 0), issued one chunk ahead of their use
        u32x4 kv[4];
        float4 u4[4];
        float lgj;
        auto load_chunk = [&](int p0) {
            const int pn = min(kMfmaChunk, plen - p0);
            const int j = s_idx[p0 + min(m, pn - 1)];
            const uint16_t* kr = K + ((rows.row0 + j) * a.Hk + hk) * kFastD + kseg;
#pragma unroll
            for (int i = 0; i < 4; ++i) kv[i] = *reinterpret_cast<const u32x4*>(kr + 8 * i);
            const float* ur = U + (size_t)j * kFastD + r0 + useg;
#pragma unroll
            for (int i = 0; i < 4; ++i) u4[i] = *reinterpret_cast<const float4*>(ur + 4 * i);
            lgj = lg[j];
        };
        load_chunk(0);
        for (int p0 = 0; p0 < plen; p0 += kMfmaChunk) {
            lds_barrier();                             // the previous chunk's operands are consumed
            {
                const float w = m < plen - p0 ? __expf(ga - lgj) : 0.f;
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const uint32_t kw = kv[e >> 3][(e >> 1) & 3] >> (16 * (e & 1));
                    s_kT[(kseg + e) * kMfmaChunk + m] = (uint16_t)(kw & 0xffffu);
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float x = w * u4[e >> 2][e & 3];
                    const uint16_t hi = __builtin_bit_cast(uint16_t, (__bf16)x);
                    const uint16_t lo = __builtin_bit_cast(uint16_t, (__bf16)(x - __uint_as_float((uint32_t)hi << 16)));
                    s_uhT[(useg + e) * kMfmaChunk + m] = hi;
                    s_ulT[(useg + e) * kMfmaChunk + m] = lo;
                }
            }
            // (LDS-only barriers: the loads just issued stay in flight over them)
            if (p0 + kMfmaChunk < plen) load_chunk(p0 + kMfmaChunk);
            lds_barrier();
            // two K = 32 halves of the chunk per accumulator tile (the second
            // only when the chunk holds more than 32 nodes: short paths)
            const int pn = min(kMfmaChunk, plen - p0);
#pragma unroll
            for (int hf = 0; hf < kMfmaChunk / 32; ++hf) {
                if (32 * hf >= pn) break;                  // uniform
                const int off = (16 * wave + ln) * kMfmaChunk + 32 * hf + 8 * lq;
                const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s_uhT + off));
                const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s_ulT + off));
#pragma unroll
                for (int tc = 0; tc < 8; ++tc) {
                    const bf16x8 ak = __builtin_bit_cast(
                        bf16x8,
                        *reinterpret_cast<const u32x4*>(s_kT + (16 * tc + ln) * kMfmaChunk + 32 * hf + 8 * lq));
                    D[tc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bh, D[tc], 0, 0, 0);
                    D[tc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bl, D[tc], 0, 0, 0);
                }
            }
        }
    }
    if (plen > 0 || a.S_in != a.S_out) {               // nothing accepted (or invalid): S_out = S_in
#pragma unroll
        for (int tc = 0; tc < 8; ++tc) *reinterpret_cast<f32x4*>(a.S_out + srow + 16 * tc) = D[tc];
    }
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a, int io, hipStream_t stream) {
    CommitArgs copy = a;
    void* args[] = {&copy};
    if (a.dk == kFastD && a.dv == kFastD) {
        // paths of up to 128 nodes: the streaming FMA kernel; longer ones: MFMA
        const void* fn = io != GDN_BF16 ? (const void*)commit_kernel_d128<GDN_F32>
                         : a.N <= 128   ? (const void*)commit_kernel_d128<GDN_BF16>
                                        : (const void*)commit_kernel_mfma;
        const unsigned grid = (unsigned)(a.B * a.Hv) * (fn == (const void*)commit_kernel_mfma ? kMfmaHalves : 1);
        return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, stream);
    }
    const void* fn = io == GDN_BF16 ? (const void*)commit_kernel<GDN_BF16>
                                    : (const void*)commit_kernel<GDN_F32>;
    dim3 grid((unsigned)(a.B * a.Hv), (unsigned)((a.dv + kRows - 1) / kRows));
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace gdn
