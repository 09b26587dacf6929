// verify_large.hip -- MFMA tree verification for d_k = d_v = 128, bf16
// q/k/v/o and trees of 129 .. 16 * NB nodes (NB = 16 or 32 blocks of 16 nodes).
//
// Same method as the small-tree kernel (page "Trees from Marginals:
// Autoregressive drafting with factorized priors", section 3: the Gram matrix,
// a tiled forward substitution and the output stage, fused), laid out for trees
// whose k / q rows and interaction tiles no longer fit in LDS together:
//  - tree_prep_kernel, one workgroup per sequence, validates the parent row
//    and writes the strict-ancestor bit rows, depth and status to the cache;
//  - verify_large_kernel, one workgroup per (sequence, value head, column
//    slice), walks the 16-node block rows t in order.  For row t it computes
//    only the Gram tiles (t, s) whose nodes have an ancestor pair (a tile
//    occupancy taken from the ancestor rows), spread over the waves, stages the
//    masked, decayed tiles in an LDS row buffer (two of them, alternating), and
//    after one barrier every wave runs row t of the blocked substitution and the
//    output stage for its 16 value columns, two node blocks per MFMA.
// k / q rows are read from global memory (L2) straight into MFMA operand
// registers; the next row's are requested before the current row's solve.
#include "gdn_common.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"

namespace gdn {

namespace {

constexpr int kPrepMaxN = 512;       // largest tree of this path
constexpr int kPrepThreads = 1024;

// Ancestor rows, depth and status of one sequence's tree, into the cache.
__global__ __launch_bounds__(kPrepThreads) void tree_prep_kernel(VerifyArgs a) {
    __shared__ uint32_t s_mask[kPrepMaxN * (kPrepMaxN / 32)];
    __shared__ int32_t s_jump[kPrepMaxN];
    __shared__ int s_flag;
    const int b = blockIdx.x, N = a.N, W = (N + 31) / 32;
    const int status = tree_build_lds(a.parent + (size_t)b * N, N, W, s_mask, s_jump, &s_flag);
    __syncthreads();
    uint32_t* gm = a.anc_mask + (size_t)b * N * W;
    for (int x = threadIdx.x; x < N * W; x += blockDim.x) gm[x] = s_mask[x];
    for (int i = threadIdx.x; i < N; i += blockDim.x)
        a.depth[(size_t)b * N + i] = status ? -1 : row_popc(s_mask + i * W, W);
    if (threadIdx.x == 0) a.status[b] = status;
}

// The index of the k-th set bit (k >= 0) of a wave-uniform 64-bit mask.
__device__ __forceinline__ int nth_bit64(uint64_t m, int k) {
    for (int i = 0; i < k; ++i) m &= m - 1;
    return __ffsll((unsigned long long)m) - 1;
}

// A/B fragment of a 16-node block of k or q straight from global memory: lane
// l gets row 16 blk + l % 16 (clamped to N - 1), columns 32 cs + 8 (l / 16)..+7.
__device__ __forceinline__ bf16x8 g_frag(const uint16_t* base, size_t row_stride, int blk,
                                         int cs, int lane, int N) {
    const int row = min(16 * blk + (lane & 15), N - 1);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                          base + (size_t)row * row_stride + 32 * cs + 8 * (lane >> 4)));
}

template <int NB, int NWV>
__global__ __launch_bounds__(64 * NWV, 1) void verify_large_kernel(VerifyArgs a, int csplit) {
    constexpr int NP = 16 * NB;                 // padded node count
    constexpr int NT = 64 * NWV;
    constexpr int NPR = NB / 2;                 // U pairs
    // -X and Y tiles of one block row, by column block s, for rows of either
    // parity; a spare tile at the end (a pair read may run 512 bytes past the
    // last tile; those lanes are zeroed before use)
    __shared__ __attribute__((aligned(16))) uint16_t s_xrow[2][NB * 256 + 256];
    __shared__ __attribute__((aligned(16))) uint16_t s_yrow[2][NB * 256 + 256];
    __shared__ __attribute__((aligned(16))) uint16_t s_dinv[2][256];
    __shared__ __attribute__((aligned(16))) float s_xd[2][256];
    __shared__ __attribute__((aligned(16))) float s_lg[NP];
    __shared__ __attribute__((aligned(16))) float s_beta[NP];
    __shared__ __attribute__((aligned(16))) int32_t s_jump[NP];
    __shared__ unsigned long long s_occ[NB];    // bit s of row t: tile (t, s), s < t, not all zero
    __shared__ int s_flag;

    const int N = a.N, Hv = a.Hv, Hk = a.Hk, G = Hv / Hk;
    const int W = (N + 31) / 32;
    const int nblk = (N + 15) / 16;
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int item = blockIdx.x;
    const int slice = item % csplit, bh = item / csplit;
    const int h = bh % Hv, b = bh / Hv, hk = h / G;
    const int col0 = slice * (16 * NWV) + 16 * wave;   // this wave's 16 value columns
    const size_t vo_row = (size_t)Hv * kD;
    const size_t vo_base = ((size_t)b * N * Hv + h) * kD;
    uint16_t* O = static_cast<uint16_t*>(a.o);
    float* Ug = a.u + ((size_t)b * Hv + h) * (size_t)N * kD;

    const int status = a.status[b];
    if (status) {                                       // invalid tree: NaN outputs
        const float qnan = __uint_as_float(0x7fc00000u);
        for (int x = lane; x < N * 16; x += 64) {
            const int i = x / 16, c = col0 + x % 16;
            O[vo_base + (size_t)i * vo_row + c] = 0x7fc0;
            Ug[(size_t)i * kD + c] = qnan;
        }
        if (slice == 0)
            for (int i = tid; i < N; i += NT) a.log_gamma[((size_t)b * Hv + h) * N + i] = qnan;
        return;
    }

    // ---- path log-gates G (synchronous pointer doubling), beta, occupancy ----
    for (int i = tid; i < NP; i += NT) {
        const bool v = i < N;
        s_jump[i] = v ? a.parent[(size_t)b * N + i] : -1;
        s_lg[i] = v ? logf(a.g[((size_t)b * N + i) * Hv + h]) : 0.f;
        s_beta[i] = v ? a.beta[((size_t)b * N + i) * Hv + h] : 0.f;
    }
    for (int t = tid; t < NB; t += NT) s_occ[t] = 0ull;
    __syncthreads();
    for (;;) {
        int nn[NP / NT > 0 ? NP / NT : 1];
        float gj[NP / NT > 0 ? NP / NT : 1];
        constexpr int PER = NP / NT > 0 ? NP / NT : 1;
        bool act = false;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * NT;
            const int j = i < NP ? s_jump[i] : -1;
            nn[k] = j >= 0 ? s_jump[j] : -1;
            gj[k] = j >= 0 ? s_lg[j] : 0.f;
            act |= j >= 0;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * NT;
            if (i < NP && s_jump[i] >= 0) {
                s_lg[i] += gj[k];
                s_jump[i] = nn[k];
            }
        }
        if (!__syncthreads_or(act)) break;
    }
    if (slice == 0)
        for (int i = tid; i < N; i += NT) a.log_gamma[((size_t)b * Hv + h) * N + i] = s_lg[i];
    {
        // occupancy: OR of the ancestor words of block t's rows, word w covering
        // column blocks 2w and 2w + 1
        const uint32_t* gm = a.anc_mask + (size_t)b * N * W;
        for (int x = tid; x < nblk * W; x += NT) {
            const int t = x / W, w = x % W;
            uint32_t acc = 0;
            for (int i = 16 * t; i < min(16 * t + 16, N); ++i) acc |= gm[(size_t)i * W + w];
            const unsigned long long bits = ((acc & 0xffffu) ? 1ull << (2 * w) : 0ull) |
                                            ((acc >> 16) ? 1ull << (2 * w + 1) : 0ull);
            if (bits) atomicOr(&s_occ[t], bits);
        }
    }

    // this wave's S0 rows (value columns col0 + l%16) as bf16 B / A operands
    bf16x8 sb[4];
    {
        const float* p = a.S0 + ((size_t)b * Hv + h) * kD * kD + (size_t)(col0 + ln) * kD + 8 * lq;
#pragma unroll
        for (int cs = 0; cs < 4; ++cs)
            sb[cs] = to_bf16x8(*reinterpret_cast<const float4*>(p + 32 * cs),
                               *reinterpret_cast<const float4*>(p + 32 * cs + 4));
    }
    __syncthreads();

    const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + ((size_t)b * N * Hk + hk) * kD;
    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + ((size_t)b * N * Hk + hk) * kD;
    const uint16_t* Vp = static_cast<const uint16_t*>(a.v) + vo_base + col0 + 4 * lq;
    const size_t kq_row = (size_t)Hk * kD;
    const uint32_t* gmask = a.anc_mask + (size_t)b * N * W;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const s16x4 zero4 = {0, 0, 0, 0};
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    const bool hi_half = lq >= 2;
    s16x4 ident;
#pragma unroll
    for (int e = 0; e < 4; ++e) ident[e] = (4 * lq + e == ln) ? (short)0x3f80 : (short)0;

    bf16x8 up[NPR];                                     // [U_2p; U_2p+1] as 16x16x32 B operands
#pragma unroll
    for (int p = 0; p < NPR; ++p) up[p] = zero8;

    // one Gram tile (t, s): masked, decayed -X / Y (bf16, tile layout) into the
    // row buffers of parity par; for s == t the diagonal X block in fp32 and its
    // inverse (16 lanes of this wave, column ln each)
    auto gram_tile = [&](int t, int s, const bf16x8 (&kt)[4], const bf16x8 (&qt)[4],
                         const bf16x8 (&ks)[4], uint32_t mword) {
        const int par = t & 1;
        f32x4 A = z, C = z;
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
            A = mfma32(ks[cs], kt[cs], A);
            C = mfma32(ks[cs], qt[cs], C);
        }
        const int i = 16 * t + ln, j0 = 16 * s + 4 * lq;
        const uint32_t bits = i < N ? (mword >> (j0 & 31)) & 15u : 0u;
        const float lgi = s_lg[i], bei = s_beta[i];
        const float4 lgj = *reinterpret_cast<const float4*>(&s_lg[j0]);
        const float lj[4] = {lgj.x, lgj.y, lgj.z, lgj.w};
        float xv[4];
        uint16_t yv[4], nxv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool anc = (bits >> e) & 1u;
            const bool self = (j0 + e == i) && i < N;
            const float d = (anc || self) ? __expf(lgi - lj[e]) : 0.f;
            xv[e] = anc ? bei * d * A[e] : 0.f;
            yv[e] = bf16_rne(d * C[e]);
            nxv[e] = bf16_rne(-xv[e]);
        }
        const int tp = a32_pos(ln, 4 * lq);
        *reinterpret_cast<uint2*>(&s_yrow[par][s * 256 + tp]) =
            make_uint2(yv[0] | ((uint32_t)yv[1] << 16), yv[2] | ((uint32_t)yv[3] << 16));
        if (s < t) {
            *reinterpret_cast<uint2*>(&s_xrow[par][s * 256 + tp]) =
                make_uint2(nxv[0] | ((uint32_t)nxv[1] << 16), nxv[2] | ((uint32_t)nxv[3] << 16));
        } else {
            *reinterpret_cast<float4*>(&s_xd[par][ln * 16 + 4 * lq]) = make_float4(xv[0], xv[1], xv[2], xv[3]);
            // (I + X_tt)^-1 by forward substitution, one column per lane; the
            // wave reads its own LDS writes (in order within a wave)
            if (lane < 16) {
                const float* xd = s_xd[par];
                float y[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float acc = (r == ln) ? 1.f : 0.f;
#pragma unroll
                    for (int m = 0; m < r; ++m) acc = fmaf(-xd[r * 16 + m], y[m], acc);
                    y[r] = acc;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) s_dinv[par][a32_pos(r, ln)] = bf16_rne(y[r]);
            }
        }
    };

    // one block row: Gram tiles, barrier, then this wave's substitution and
    // outputs.  kt / qt / vt are row t's operands (requested a row earlier);
    // kn / qn / vn receive row t + 1's.
    auto do_row = [&](int t, const bf16x8 (&kt)[4], const bf16x8 (&qt)[4], uint2 vt,
                      bf16x8 (&kn)[4], bf16x8 (&qn)[4], uint2& vn) {
        const int par = t & 1;
        // (readfirstlane returns a signed int: widen through uint32_t, and keep
        // only column blocks 0 .. t)
        const unsigned long long occ =
            (((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(s_occ[t] >> 32)) << 32) |
             (unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)s_occ[t])) &
            ((2ull << t) - 1ull);
        const unsigned long long full = occ | (1ull << t);
        const int ntile = __popcll(full);
        // this wave's tiles of the row, two at a time (both tiles' k rows and
        // ancestor words requested before either is computed)
        for (int m = wave; m < ntile; m += 2 * NWV) {
            const int s0 = nth_bit64(full, m);
            const bool two = m + NWV < ntile;
            const int s1 = two ? nth_bit64(full, m + NWV) : s0;
            bf16x8 k0[4], k1[4];
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
                k0[cs] = g_frag(Kb, kq_row, s0, cs, lane, N);
                k1[cs] = g_frag(Kb, kq_row, s1, cs, lane, N);
            }
            const int ii = min(16 * t + ln, N - 1);
            const uint32_t w0 = gmask[(size_t)ii * W + ((16 * s0 + 4 * lq) >> 5)];
            const uint32_t w1 = gmask[(size_t)ii * W + ((16 * s1 + 4 * lq) >> 5)];
            gram_tile(t, s0, kt, qt, k0, w0);
            if (two) gram_tile(t, s1, kt, qt, k1, w1);
        }
        lds_barrier();                                  // row t's tiles and inverse are published
        // row t + 1's operands (the last row re-reads its own: harmless)
        const int tn = min(t + 1, nblk - 1);
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
            kn[cs] = g_frag(Kb, kq_row, tn, cs, lane, N);
            qn[cs] = g_frag(Qb, kq_row, tn, cs, lane, N);
        }
        vn = *reinterpret_cast<const uint2*>(Vp + (size_t)min(16 * tn + ln, N - 1) * vo_row);

        // ---- substitution and outputs for row t, this wave's 16 columns ----
        const uint16_t* xr = s_xrow[par];
        const uint16_t* yr = s_yrow[par];
        f32x4 pk = z, pqT = z;
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
            pk = mfma32(kt[cs], sb[cs], pk);            // [node][r]
            pqT = mfma32(sb[cs], qt[cs], pqT);          // [r][node]
        }
        f32x4 R;
        {
            const f32x4 vd = mfma16(__builtin_bit_cast(s16x4, vt), ident, z);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int i = 16 * t + 4 * lq + m;
                R[m] = s_beta[i] * (vd[m] - __expf(s_lg[i]) * pk[m]);
            }
        }
        // R_t += sum_{s<t} (-X_ts) U_s over occupied tiles, two blocks per MFMA
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
            const int s = 2 * p;
            if (s < t) {
                const bool o0 = (occ >> s) & 1ull;
                const bool o1 = s + 1 < t && ((occ >> (s + 1)) & 1ull);
                if (o0 || o1) {
                    bf16x8 nx = *reinterpret_cast<const bf16x8*>(xr + s * 256 + lane * 8);
                    if (!(hi_half ? o1 : o0)) nx = zero8;
                    R = mfma32(nx, up[p], R);
                }
            }
        }
        const bf16x8 di = *reinterpret_cast<const bf16x8*>(s_dinv[par] + (ln + 16 * (lq & 1)) * 8);
        s16x4 rh, rl;
        split4(R, rh, rl);
        const bf16x8 rr = stack_pair(rh, rl);
        const f32x4 U = mfma32(di, rr, z);
        const f32x4 UT = mfma32(rr, di, z);
        const s16x4 ut = to_bf16x4(U);
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
            if (p == (t >> 1)) {
                if (t & 1)
                    up[p] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, up[p]) |
                                                           __builtin_bit_cast(u32x4, stack_pair(zero4, ut)));
                else
                    up[p] = stack_pair(ut, zero4);
            }
        }
        const int node = 16 * t + ln;
        if (node < N) *reinterpret_cast<f32x4*>(Ug + (size_t)node * kD + col0 + 4 * lq) = UT;
        // O_t^T = e^G P_Q^T + sum_{s<=t} U_s^T Y_ts^T over occupied tiles
        f32x4 Oc = z;
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
            const int s = 2 * p;
            if (s <= t) {
                const bool o0 = s == t || ((occ >> s) & 1ull);
                const bool o1 = s + 1 == t || (s + 1 < t && ((occ >> (s + 1)) & 1ull));
                if (o0 || o1) {
                    bf16x8 yt = *reinterpret_cast<const bf16x8*>(yr + s * 256 + lane * 8);
                    if (!(hi_half ? o1 : o0)) yt = zero8;
                    Oc = mfma32(up[p], yt, Oc);
                }
            }
        }
        if (node < N) {
            const float egn = __expf(s_lg[node]);
            f32x4 OT;
#pragma unroll
            for (int m = 0; m < 4; ++m) OT[m] = egn * pqT[m] + Oc[m];
            const uint32_t lo = (uint32_t)bf16_rne(OT[0]) | ((uint32_t)bf16_rne(OT[1]) << 16);
            const uint32_t hi = (uint32_t)bf16_rne(OT[2]) | ((uint32_t)bf16_rne(OT[3]) << 16);
            *reinterpret_cast<uint2*>(O + vo_base + (size_t)node * vo_row + col0 + 4 * lq) = make_uint2(lo, hi);
        }
    };

    // rows in pairs, the operand registers alternating (no copies of loads in flight)
    bf16x8 ka[4], qa[4], kb2[4], qb2[4];
    uint2 va, vb;
#pragma unroll
    for (int cs = 0; cs < 4; ++cs) {
        ka[cs] = g_frag(Kb, kq_row, 0, cs, lane, N);
        qa[cs] = g_frag(Qb, kq_row, 0, cs, lane, N);
    }
    va = *reinterpret_cast<const uint2*>(Vp + (size_t)min(ln, N - 1) * vo_row);
    for (int t = 0; t < nblk; t += 2) {
        do_row(t, ka, qa, va, kb2, qb2, vb);
        if (t + 1 < nblk) do_row(t + 1, kb2, qb2, vb, ka, qa, va);
    }
}

}  // namespace

bool verify_large_supported(const VerifyArgs& a, int io) {
    return io == GDN_BF16 && a.dk == kD && a.dv == kD && a.N > 128 && a.N <= kPrepMaxN;
}

hipError_t launch_verify_large(const VerifyArgs& a, int io, hipStream_t stream) {
    (void)io;
    VerifyArgs copy = a;
    void* pargs[] = {&copy};
    hipError_t e = hipLaunchKernel((const void*)tree_prep_kernel, dim3((unsigned)a.B), dim3(kPrepThreads),
                                   pargs, 0, stream);
    if (e != hipSuccess) return e;
    // two column slices of 64 value columns per (sequence, value head), four
    // waves each: a wave holds up to 32 stacked U pairs and may use the whole
    // register file of its SIMD
    int csplit = 2;
    const void* fn = a.N <= 256 ? (const void*)verify_large_kernel<16, 4> : (const void*)verify_large_kernel<32, 4>;
    void* args[] = {&copy, &csplit};
    return hipLaunchKernel(fn, dim3((unsigned)(a.B * a.Hv * csplit)), dim3(256), args, 0, stream);
}

}  // namespace gdn
