// verify_large.hip -- MFMA tree verification for d_k = d_v = 128, bf16
// q/k/v/o and trees of 129 .. 16 * NB nodes (NB = 16, 32 or 64 blocks of 16 nodes).
//
// Same method as the small-tree kernel (page "Trees from Marginals:
// Autoregressive drafting with factorized priors", section 3: the Gram matrix,
// a tiled forward substitution and the output stage, fused), laid out for
// trees whose interaction tiles do not fit in LDS.  One workgroup per
// (sequence, value head, 64-column slice), twelve waves in two roles that
// meet through LDS counters, with no barrier after the setup:
//
//  * setup (all waves): the parent row is checked; one wave relabels the
//    tree's nodes in preorder (every subtree one run of positions, so
//    ancestry is an interval test and a block row's ancestors sit in few
//    column blocks) while another sums the path log-gates, both by pointer
//    jumping within the wave; the tree's workgroups share writing its
//    ancestor rows, depths and status.  The workgroup's global inputs are
//    requested first (for trees of up to 256 nodes the k rows, stored into
//    LDS at its end), so their latency overlaps it; its barriers order LDS
//    only.
//  * producers (waves 4 .. 11): the work of all block rows as one row-major
//    list of items, each producer's first dealt round robin and the rest
//    claimed in order, each item's global operands requested one item
//    ahead.  A row's first item forms the diagonal block's inverse
//    D_t = (I + X_tt)^-1 (fp32 substitution, kept bf16) and its output tile
//    Y_tt (and, without k in LDS, the row's right-hand sides); the others form, for a few occupied column blocks s, the tiles
//    -X_ts and Y_ts from one read of k_s.  Tiles go to a ring of LDS slots,
//    D_t to a table; a per-row counter says when the row is complete.
//  * solve (waves 0 .. 3, 16 value columns each): row by row, the
//    right-hand side R_t = diag(beta)(V_t - diag(e^G) K_t S0^T) and the
//    substitution U_t = D_t (R_t - sum_s X_ts U_s), the row's outputs
//    O_t = e^G Q_t S0^T + sum_{s <= t} Y_ts U_s, then the ring slots are
//    released.  A column group needs no other group's U, so the four solve
//    waves never wait for each other.
//
// Inputs are gathered and outputs written at the caller's node indices.
#include "gdn_common.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"


namespace gdn {

namespace {

constexpr int kLargeMaxN = 1024;     // largest tree of this path
constexpr int kLargeWaves = 12;
constexpr int kLargeThreads = 64 * kLargeWaves;
constexpr int kSolveWaves = 4;       // one 16-column group each: 64 columns per workgroup
constexpr int kProducers = kLargeWaves - kSolveWaves;

// buffer resources for stores that must not branch on a lane's validity: a
// lane's store past the buffer is dropped
constexpr int kBufferFlags = 0x00020000;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// x of lane k of each lane quad, to all four lanes (k a compile-time value
// once the caller's loop is unrolled).
__device__ __forceinline__ float quad_bcast(float x, int k) {
    const int v = __float_as_int(x);
    switch (k) {
        case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false));
        case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false));
        case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xaa, 0xf, 0xf, false));
        default: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xff, 0xf, 0xf, false));
    }
}

// Spin until *f >= v.  The flags live in LDS and only grow; a flag's writer
// never waits for its readers' later work, so every wait ends.
__device__ __forceinline__ void wait_flag_ge(int* f, int v) {
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < v)
        __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
}
// This wave's LDS reads and writes are complete, then lane 0 stores v.
__device__ __forceinline__ void publish_set(int* f, int v, int lane) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// (Masked entries are computed for every lane and then selected, so no lane
// takes a branch: e^(G_i - G_j) is taken of min(G_i - G_j, 0), which leaves
// every ancestor pair's value unchanged -- the path of i contains j's, and
// every gate is at most 1 -- and keeps the discarded ones finite.)

// A 16x16 bf16 tile as a 16x16x16 A operand: lane l holds row l % 16,
// columns 4 (l / 16) .. +3, one 8-byte word per lane.  Element (r, c) in
// halfwords:
__device__ __forceinline__ int a16_pos(int r, int c) { return (r + 16 * (c >> 2)) * 4 + (c & 3); }

// 16-byte chunk c of 128-element bf16 row r in LDS, XOR-swizzled by the row's
// low bits so the 16 rows of a fragment read fall in distinct banks.
__device__ __forceinline__ int row_chunk(int r, int c) { return r * kD + ((c ^ (r & 15)) << 3); }

template <int NB>
struct LargeShape {
    static constexpr int NP = 16 * NB;
    static constexpr bool KLDS = NB <= 16;              // the k rows sit in LDS
    static constexpr int C = KLDS ? 2 : 1;              // occupied column blocks per producer item
    // words of a children row (past 512 nodes there is no children table: a
    // node's next sibling comes from a scan of the later nodes' parents)
    static constexpr int WC = NB <= 32 ? NP / 32 : 0;
    static constexpr int SCRATCH = ((NP + 1) * WC + (NP + 2) + 8 * NP) * 4;   // the preorder's
    // A row's slots: when k is not in LDS, first its right-hand sides R_t and
    // e^G Q_t S0^T (fp32, two slots per column group each) and D_t (HDR
    // slots in all); then its -X tiles and its Y tiles (the diagonal block's
    // last).  Rows with a header take an even number of slots, so two-slot
    // objects never wrap.
    static constexpr int HDR = KLDS ? 0 : 17;
    static constexpr int NFIX = 1;                      // items of a row before its occupied blocks'

    static constexpr int RING = NB <= 16 ? 84 : NB <= 32 ? 112 : 184;   // 512-byte tile slots
    // block rows of U kept in LDS by each solve wave: all of them up to 512
    // nodes; past that UW slots, each held from its row until the last row
    // that reads it (so that the ring takes the rest)
    static constexpr int UW = NB <= 32 ? NB : 8;
    static constexpr int BIG = RING * 512 > SCRATCH ? RING * 512 : SCRATCH;
    // items: per row one for the diagonal block, without k in LDS one for the
    // right-hand sides, and one per C occupied blocks
    static constexpr int ITEMS = NFIX * NB + (C == 1 ? NB * (NB - 1) / 2 : (NB / 2) * (NB / 2));
};

// FUSED: the previous tree's commit (page "Trees from Marginals", section 3:
// the deferred state commit) runs first in the same launch; its state rows
// become this verification's S0 without a trip through memory.
template <int NB, bool FUSED>
__global__ __launch_bounds__(kLargeThreads, 1) void verify_large_kernel(VerifyArgs a, CommitArgs c, int units) {
    using L = LargeShape<NB>;
    constexpr int NP = L::NP;
    constexpr int NT = kLargeThreads;
    constexpr bool KLDS = L::KLDS;
    constexpr int C = L::C;
    constexpr int WC = L::WC;
    constexpr int SCRATCH = L::SCRATCH;
    constexpr int BIG = L::BIG;
    constexpr int RING = L::RING;
    constexpr int PL = (NP + NT - 1) / NT;              // tree entries per thread
    constexpr int HDR = L::HDR;
    constexpr int NFIX = L::NFIX;
    static_assert(2 * (NB - 1) + 1 + HDR <= RING && RING % 2 == 0, "a row's slots fit the ring");
    static_assert(NB <= 64 && NB % 2 == 0, "block rows in one wave's lanes");
    constexpr int UW = L::UW;
    // the ring of tile slots (8 bytes per lane each); during the setup the
    // preorder's scratch
    __shared__ __attribute__((aligned(16))) uint2 s_big[BIG / 8];
    __shared__ __attribute__((aligned(16))) uint16_t s_k[KLDS ? NP * kD : 8];   // k rows, node order
    __shared__ __attribute__((aligned(16))) uint2 s_u[UW][kSolveWaves][64];   // U_t, bf16 B operands
    __shared__ int s_uslot[UW < NB ? NB : 1];          // (with slots) row t's slot of s_u, -1: none
    __shared__ __attribute__((aligned(16))) uint2 s_d[KLDS ? NB : 1][64];    // D_t, bf16 A operands (else in the ring)
    __shared__ __attribute__((aligned(16))) uint16_t s_s0[KLDS ? 8 : 64 * kD];   // the slice's S0 rows, bf16
    __shared__ __attribute__((aligned(16))) float s_xd[kProducers][256];     // each producer's X_tt, fp32 [col][row]
    __shared__ __attribute__((aligned(16))) float s_lg[NP];
    __shared__ __attribute__((aligned(16))) float s_beta[NP];
    __shared__ __attribute__((aligned(16))) int32_t s_jump[NP];
    __shared__ uint16_t s_perm[NP];                     // position -> node
    __shared__ __attribute__((aligned(8))) int16_t s_last[NP];   // position of the last descendant
    __shared__ int16_t s_hop[NP];                       // nodes on the path to the root (depth + 1)
    __shared__ __attribute__((aligned(16))) int s_mlast[NB];   // largest s_last of each block
    __shared__ __attribute__((aligned(16))) uint8_t s_tcol[NB][NB];   // row t's occupied blocks s < t, ascending
    __shared__ int s_tn[NB];                            // their number
    __shared__ __attribute__((aligned(16))) int s_gslot[NB + 4];   // first slot of row t, counted over all rows
    __shared__ int s_rstar[NB];                         // rows released before row t's slots are free
    __shared__ uint16_t s_items[L::ITEMS];              // producer items: row | (item of the row << 8)
    __shared__ int s_nitems;
    __shared__ int s_claim;                             // producer items claimed past the first kProducers
    __shared__ int s_done[NB];                          // row t's tiles and parts finished (complete at s_tn[t] + NFIX)
    __shared__ int s_oready[kSolveWaves];               // rows finished by each solve wave
    __shared__ int s_bad;                               // first node with an invalid parent
    __shared__ int s_notchain;                          // some node's parent is not the node before it
    __shared__ int s_more[3];                           // per-round "not done" flags of the jumping loops

    const int N = a.N, Hv = a.Hv, Hk = a.Hk, G = Hv / Hk;
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // workgroups are dealt to the 8 XCDs round robin: the two slices of a
    // (sequence, head) are 8 workgroups apart, on one XCD, sharing its L2
    const int bid = blockIdx.x;
    const int unit = 8 * (bid >> 4) + (bid & 7), slice = (bid >> 3) & 1;
    if (unit >= units) return;
    const int h = unit % Hv, b = unit / Hv, hk = h / G;
    const int cbase = 64 * slice;                       // the workgroup's first value column
    // this tree's rows in the node arrays (n nodes); the cache keeps N rows per tree
    const SeqRows rows = seq_rows(a.offsets, b, N);
    const int n = max(rows.n, 0);
    const int nblk = (n + 15) / 16;
    const size_t vo_row = (size_t)Hv * kD;
    const size_t vo_base = (rows.row0 * Hv + h) * kD;
    uint16_t* O = static_cast<uint16_t*>(a.o);
    float* Ug = a.u + ((size_t)b * Hv + h) * (size_t)N * kD;
    const bool solver = wave < kSolveWaves;
    const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + (rows.row0 * Hk + hk) * kD;
    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + (rows.row0 * Hk + hk) * kD;
    const size_t kq_row = (size_t)Hk * kD;

    // ---- the workgroup's inputs, requested before anything waits ----
    // parent, g, beta of the tree's nodes
    int par_r[PL];
    float g_r[PL], beta_r[PL];
#pragma unroll
    for (int k = 0; k < PL; ++k) {
        const int i = tid + k * NT;
        const bool v = i < n;
        par_r[k] = v ? a.parent[rows.row0 + i] : -1;
        g_r[k] = v ? a.g[(rows.row0 + i) * Hv + h] : 1.f;
        beta_r[k] = v ? a.beta[(rows.row0 + i) * Hv + h] : 0.f;
    }
    // a solve wave's 16 S0 rows (fp32; its bf16 operands are formed after the
    // setup): lane (r, q) takes row cbase + 16 wave + r, columns 32 cs + 8 q .. +7
    // (For a chain the same registers bring each producer's first q and v
    // rows during the setup: see the chain path.)
    float4 s0_r[8];
    if (!FUSED && KLDS && solver) {
        const float* S0p =
            a.S0 + ((size_t)b * Hv + h) * kD * kD + (size_t)(cbase + 16 * wave + ln) * kD + 8 * lq;
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
            s0_r[2 * cs] = *reinterpret_cast<const float4*>(S0p + 32 * cs);
            s0_r[2 * cs + 1] = *reinterpret_cast<const float4*>(S0p + 32 * cs + 4);
        }
    }
    // without k in LDS: the slice's 64 S0 rows (fp32), converted into LDS at
    // the end of the setup for the producers
    constexpr int S0L = KLDS ? 1 : (64 * kD / 4 + NT - 1) / NT;   // float4 loads per thread
    float4 s0s[S0L];
    if constexpr (!KLDS && !FUSED) {
        const float* S0p = a.S0 + ((size_t)b * Hv + h) * kD * kD + (size_t)cbase * kD;
#pragma unroll
        for (int k = 0; k < S0L; ++k) {                 // (float4 index in the 64 x 128 slice, clamped)
            const int x = min(tid + k * NT, 64 * kD / 4 - 1);
            s0s[k] = *reinterpret_cast<const float4*>(S0p + 4 * x);
        }
    }
    // k rows of the tree (node order, rows past the tree copy row n - 1) into
    // registers, written to LDS at the end of the setup (a direct-to-LDS
    // load would make the compiler wait for it before the setup's first LDS
    // access): one 1 KB unit is four rows, lane l taking row 4u + l / 16 and
    // its logical chunk (l % 16) ^ (row & 15), so the store is one contiguous
    // 16-byte write per lane
    // (with the commit fused, requested after the commit's first requests:
    // requests retire in order, so the commit would otherwise wait for them)
    constexpr int KI = KLDS ? (NP / 4 + kLargeWaves - 1) / kLargeWaves : 1;
    u32x4 k_r[KI];
    auto request_k = [&]() __attribute__((always_inline)) {
        if constexpr (KLDS) {
#pragma unroll
            for (int kk = 0; kk < KI; ++kk) {
                const int u = min(wave + kk * kLargeWaves, NP / 4 - 1);
                const int row = 4 * u + (lane >> 4), pc = lane & 15;
                const int srow = min(row, max(n - 1, 0));
                k_r[kk] = *reinterpret_cast<const u32x4*>(Kb + (size_t)srow * kq_row + ((pc ^ (row & 15)) << 3));
            }
        }
    };
    if constexpr (!FUSED) request_k();
    // (the loaded values are used only below: their arithmetic may not be
    // moved up to the loads, where it would wait for them before the other
    // requests are out)
#pragma unroll
    for (int k = 0; k < PL; ++k) asm volatile("" : "+v"(par_r[k]), "+v"(g_r[k]), "+v"(beta_r[k]));
    // ---- the previous tree's commit (fused form) ----
    // S_a = e^(G_a) S_prev + sum_{j on a's path} e^(G_a - G_j) u_j k_j^T for
    // the slice's 64 state rows, a the previous tree's accepted node and G, u
    // its cached path log-gates and writes; as in the separate commit, as
    // D^T = e^(G_a) D_in^T + K_P^T (diag(w) U_P), with the weighted u split
    // into bf16 hi + lo parts (about 16 mantissa bits).  Solve wave g forms
    // its rows c0 .. c0 + 15 alone, 16 path nodes at a time, before the
    // verification's setup: its eight accumulator tiles (lane (r, q): row
    // c0 + r, columns 16 tc + 4 q .. +3) take K^T and W tiles that the
    // matrix cores themselves transpose, an exact product of the tiles as
    // read (nodes in rows) with an identity or column selection, so nothing
    // goes through LDS and no wave waits for another.  The rows go to the
    // new state and, as bf16, become this launch's S0 (the solve waves'
    // operands with k in LDS, the producers' table without).
    bf16x8 s0g[4];
    if constexpr (FUSED) {
        // The path comes through the scalar cache (uniform addresses in the
        // constant address space): a vector load here would wait for every
        // vector request above it, the k rows included.
        typedef const __attribute__((address_space(4))) uint32_t* cu32;
        typedef const __attribute__((address_space(4))) float* cf32;
        typedef const __attribute__((address_space(4))) int32_t* ci32;
        int* s_path = reinterpret_cast<int*>(reinterpret_cast<char*>(s_big) + BIG) - NP;
        const int Wc = (N + 31) / 32;
        const int acc = ((ci32)c.accepted)[b];
        const SeqRows prow = seq_rows(c.offsets, b, N);
        const bool cvalid = ((ci32)c.status)[b] == 0 && prow.n >= 0 && acc >= -1 && acc < prow.n;
        const int aw = acc < 0 ? 0 : acc;
        cu32 arow = (cu32)(c.anc_mask + ((size_t)b * N + aw) * Wc);   // the accepted node's ancestor row
        const float* lgp = c.log_gamma + ((size_t)b * Hv + h) * N;
        const float ga = ((cf32)lgp)[aw];
        if (wave == 0) {
            // strict ancestors ascending, then a: word w's set bits at
            // positions counted from the words before it, lane l taking bit l
            int base = 0;
            for (int w = 0; w < Wc; ++w) {
                const uint32_t x = arow[w];
                if (cvalid && acc >= 0 && lane < 32 && ((x >> lane) & 1u))
                    s_path[base + __popc(x & ((1u << lane) - 1u))] = 32 * w + lane;
                base += __popc(x);
            }
            const int plen = !cvalid ? -1 : acc < 0 ? 0 : base + 1;
            if (lane == 0) {
                if (plen > 0) s_path[plen - 1] = acc;
                s_more[0] = plen;                       // (shared with the other waves below)
            }
        }
        lds_barrier();
        static_assert(64 * kD * 2 + NP * 4 <= BIG, "the path fits past the temporary S0 rows");
        const int plen = s_more[0];
        if (!solver || plen <= 0) request_k();
        if (h == 0 && slice == 0) {
            int32_t* pb = c.path + prow.row0;
            for (int m = tid; m < prow.n; m += NT) pb[m] = m < plen ? s_path[m] : -1;
            if (tid == 0) c.path_len[b] = plen;
        }
        if (solver) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const int g = wave, c0 = cbase + 16 * g;
            const size_t srow = ((size_t)b * Hv + h) * kD * kD + (size_t)(c0 + ln) * kD + 4 * lq;
            f32x4 cD[8];
            const float dec = plen > 0 ? __expf(ga) : 1.f;
#pragma unroll
            for (int tc = 0; tc < 8; ++tc) cD[tc] = dec * *reinterpret_cast<const f32x4*>(c.S_in + srow + 16 * tc);
            if (plen > 0) {
                const uint16_t* Kp = static_cast<const uint16_t*>(c.k) + (prow.row0 * Hk + hk) * kD;
                const float* Up = c.u + ((size_t)b * Hv + h) * (size_t)N * kD + c0;
                // a group of 16 path nodes, node ln of lane (ln, q): k columns
                // 32 w + 8 q .. +7 (w = 0 .. 3), u columns c0 + 4 q .. +3, its
                // log-gate (nodes past the path re-read its last, weight 0)
                struct Grp {
                    u32x4 k[4];
                    float4 u;
                    float lg;
                };
                auto load_grp = [&](int g0, Grp& G) __attribute__((always_inline)) {
                    const int m = min(g0 + ln, plen - 1);
                    const int j = s_path[m];
                    const uint16_t* kr = Kp + (size_t)j * kq_row + 8 * lq;
#pragma unroll
                    for (int w = 0; w < 4; ++w) G.k[w] = *reinterpret_cast<const u32x4*>(kr + 32 * w);
                    G.u = *reinterpret_cast<const float4*>(Up + (size_t)j * kD + 4 * lq);
                    G.lg = lgp[j];
                    // (no memory access may move across: the requests stay
                    // here, a group ahead of their use, and nothing waits)
                    asm volatile("" ::: "memory");
                };
                // identity (16 x 16) and the two 16-column selections of a
                // 32-column window, as B operands
                s16x4 ident;
#pragma unroll
                for (int e = 0; e < 4; ++e) ident[e] = (4 * lq + e == ln) ? (short)0x3f80 : (short)0;
                bf16x8 sel[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int e = 0; e < 8; ++e) sel[hh][e] = (__bf16)((8 * lq + e == 16 * hh + ln) ? 1.f : 0.f);
                auto apply = [&](int g0, const Grp& G) __attribute__((always_inline)) {
                    // K^T tiles: lane (c, q) holds k of nodes 4q .. 4q+3 at column 16 tc + c
                    s16x4 kt[8];
#pragma unroll
                    for (int w = 0; w < 4; ++w)
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
                            kt[2 * w + hh] = to_bf16x4(mfma32(__builtin_bit_cast(bf16x8, G.k[w]), sel[hh], z));
                    // W tiles (weighted u, hi and lo): lane (r, q) holds nodes 4q .. 4q+3 of row c0 + r
                    const float w = g0 + ln < plen ? __expf(ga - G.lg) : 0.f;
                    const f32x4 wu = {w * G.u.x, w * G.u.y, w * G.u.z, w * G.u.w};
                    s16x4 whi, wlo;
                    split4(wu, whi, wlo);
                    const s16x4 bh = to_bf16x4(mfma16(whi, ident, z));
                    const s16x4 bl = to_bf16x4(mfma16(wlo, ident, z));
#pragma unroll
                    for (int tc = 0; tc < 8; ++tc) cD[tc] = mfma16(kt[tc], bl, mfma16(kt[tc], bh, cD[tc]));
                };
                // three groups in flight: each group's requests go out two
                // groups ahead of its products
                Grp gp0, gp1, gp2;
                load_grp(0, gp0);
                load_grp(min(16, plen - 1), gp1);
                request_k();
                for (int g0 = 0; g0 < plen; g0 += 48) {
                    load_grp(min(g0 + 32, plen - 1), gp2);
                    apply(g0, gp0);
                    if (g0 + 16 >= plen) break;
                    load_grp(min(g0 + 48, plen - 1), gp0);
                    apply(g0 + 16, gp1);
                    if (g0 + 32 >= plen) break;
                    load_grp(min(g0 + 64, plen - 1), gp1);
                    apply(g0 + 32, gp2);
                }
            }
            // (in place, S_in = S_out: each workgroup reads its rows before writing them)
            if (plen > 0 || c.S_in != c.S_out) {
#pragma unroll
                for (int tc = 0; tc < 8; ++tc) *reinterpret_cast<f32x4*>(c.S_out + srow + 16 * tc) = cD[tc];
            }
            // this wave's rows as bf16 through LDS (its own rows: no barrier
            // needed; the other waves touch the area only after the next
            // barrier, which this wave reaches only once done with it)
            uint16_t* s0t = KLDS ? reinterpret_cast<uint16_t*>(s_big) : s_s0;   // [64][128] bf16, chunks swizzled
#pragma unroll
            for (int tc = 0; tc < 8; ++tc) {
                uint2 w;
                w.x = (uint32_t)bf16_rne(cD[tc][0]) | ((uint32_t)bf16_rne(cD[tc][1]) << 16);
                w.y = (uint32_t)bf16_rne(cD[tc][2]) | ((uint32_t)bf16_rne(cD[tc][3]) << 16);
                *reinterpret_cast<uint2*>(s0t + row_chunk(16 * g + ln, 2 * tc + (lq >> 1)) + 4 * (lq & 1)) = w;
            }
            if constexpr (KLDS) {
#pragma unroll
                for (int cs = 0; cs < 4; ++cs)
                    s0g[cs] = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4*>(s0t + row_chunk(16 * g + ln, 4 * cs + lq)));
            }
        }
    }
    // (Every barrier of the setup orders LDS only: the global loads above and
    // the cache rows stored below stay in flight across it.)
    // tree check, the same in every workgroup of the tree: 0, or one plus the
    // first node whose parent is outside [-1, i); -1 for rows past the
    // batch's offsets.  For an invalid or empty tree one workgroup publishes
    // zero ancestor rows, depth -1 and the status; a valid tree's rows and
    // depths are shared out once its preorder is known.
    const int W = (N + 31) / 32;
    const bool writer = h == 0 && slice == 0;
    uint32_t* gm = a.anc_mask + (size_t)b * N * W;
    if (tid == 0) {
        s_bad = 0x7fffffff;
        s_notchain = 0;
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < PL; ++k) {
        const int i = tid + k * NT;
        if (i < n && (par_r[k] < -1 || par_r[k] >= i)) atomicMin(&s_bad, i);
    }
    lds_barrier();
    const int status = rows.n < 0 ? -1 : s_bad == 0x7fffffff ? 0 : s_bad + 1;
    if (writer && (status || n == 0)) {
        for (int x = tid; x < N * W; x += NT) gm[x] = 0u;
        for (int r = tid; r < N; r += NT) a.depth[(size_t)b * N + r] = -1;
        if (tid == 0) a.status[b] = status;
    }
    if (status) {                                       // invalid tree: NaN outputs
        const float qnan = __uint_as_float(0x7fc00000u);
        if (solver)
            for (int x = lane; x < N * 16; x += 64) {
                const int i = x >> 4, col = cbase + 16 * wave + (x & 15);
                if (i < n) O[vo_base + (size_t)i * vo_row + col] = 0x7fc0;
                Ug[(size_t)i * kD + col] = qnan;
            }
        if (slice == 0)
            for (int i = tid; i < N; i += NT) a.log_gamma[((size_t)b * Hv + h) * N + i] = qnan;
        return;
    }
    if (n == 0) return;                                 // an empty tree: nothing to verify

    // ---- a preorder of the tree, path log-gates G, beta, tile occupancy ----
    // In a preorder (children in index order) j is a strict ancestor of i
    // exactly when j < i <= last(j), last(j) the position of j's last
    // descendant, so a block row's ancestors sit in few column blocks (a
    // random tree's rows touch most blocks in the caller's order) and the
    // tile masks need no ancestor rows.  Outputs stay in the caller's order.
    // Scratch while it is built: the ring area.
    uint32_t* s_cm = reinterpret_cast<uint32_t*>(s_big);          // [NP + 1][WC]; row NP: the roots
    int32_t* s_fc = reinterpret_cast<int32_t*>(s_cm + (NP + 1) * WC);   // [NP + 1] first child (NP: none)
    // pointer-jumping entries, each read and written as one 8-byte word:
    int2* s_na = reinterpret_cast<int2*>(s_fc + (NP + 2));   // [NP] (node after the subtree: n none, -1 pending; link)
    int2* s_gj = s_na + NP;                             // [2][NP] (link | hops << 16, summed log-gate bits)
    int2* s_rs = s_gj + 2 * NP;                         // [NP] (list distance to the last node, list link)
    static_assert(SCRATCH <= BIG, "preorder scratch fits the ring area");
    bool not_chain = false;                             // a chain is its own preorder
#pragma unroll
    for (int k = 0; k < PL; ++k) {
        const int i = tid + k * NT;
        if (i < NP) {
            const bool v = i < n;
            not_chain |= v && par_r[k] != i - 1;
            s_jump[i] = v ? par_r[k] : -1;
            s_lg[i] = v ? logf(g_r[k]) : 0.f;
            s_beta[i] = v ? beta_r[k] : 0.f;
            s_perm[i] = (uint16_t)min(i, max(n - 1, 0));
            s_last[i] = v ? (int16_t)(n - 1) : (int16_t)-1;
            s_hop[i] = v ? (int16_t)1 : (int16_t)0;
        }
    }
    for (int x = tid; x < (NP + 1) * WC; x += NT) s_cm[x] = 0u;
    for (int x = tid; x <= NP; x += NT) s_fc[x] = NP;
    // (without the children table: per parent, NP for the roots, its number
    // of children, then where they start in a list of the nodes by parent;
    // before the pointer jumping, in its area)
    int* const s_cnt = reinterpret_cast<int*>(s_gj);    // [NP + 2]
    if constexpr (WC == 0)
        for (int x = tid; x <= NP + 1; x += NT) s_cnt[x] = 0;
    if (tid < NB) s_done[tid] = 0;
    if (tid == 0) s_claim = 0;
    if (tid < kSolveWaves) s_oready[tid] = 0;
    if (tid < 3) s_more[tid] = 0;
    // a chain skips the construction (nt = 0): the identity and last = n - 1
    if (not_chain) s_notchain = 1;
    lds_barrier();
    const int nt = s_notchain ? n : 0;
    // A chain's first operands (the chain path below) are requested during
    // the setup, so that they arrive meanwhile: each producer's first row,
    // each solve wave's state rows.
    const int clast = max(n - 1, 0);
    const uint32_t lane_col = 16u * lq;
    // k / q fragment of block t of a chain (node = position): lane (r, q)
    // holds row 16 t + r (clamped), columns 32 cs + 8 q .. +7
    auto cfrag = [&](const uint16_t* base, int t, int cs) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)min(16 * t + ln, clast) * (uint32_t)(kq_row * 2) + lane_col + 64u * cs;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              reinterpret_cast<const char*>(base) + off));
    };
    struct DiagOps {
        bf16x8 kt[KLDS ? 1 : 4];                        // (without k in LDS) k of the row
        bf16x8 qt[4];
        u32x4 vt[2];                                    // lane (r, q): node r, columns 16 q .. +15
    };
    const uint16_t* const Vsl = static_cast<const uint16_t*>(a.v) + vo_base + cbase;
    auto dfetch = [&](int t, DiagOps& o) __attribute__((always_inline)) {
        t = min(t, max((n + 15) / 16 - 1, 0));
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
            o.qt[cs] = cfrag(Qb, t, cs);
            if constexpr (!KLDS) o.kt[cs] = cfrag(Kb, t, cs);
        }
        const uint16_t* vr = Vsl + (size_t)min(16 * t + ln, clast) * vo_row + 16 * lq;
        o.vt[0] = *reinterpret_cast<const u32x4*>(vr);
        o.vt[1] = *reinterpret_cast<const u32x4*>(vr + 8);
    };
    if constexpr (WC == 0) {
        // Next siblings from a counting sort of the nodes by parent: each
        // node takes a place in its parent's bucket in any order, then its
        // rank by index among the bucket's nodes (all of which read the
        // bucket's same words) fixes the order; the next sibling is the
        // bucket's next node.
        int* const s_tmp = s_cnt + NP + 2;              // [NP] nodes by parent, any order
        int* const s_srt = s_tmp + NP;                  // [NP] nodes by parent, ascending
        int* const s_ws = reinterpret_cast<int*>(s_rs); // the scan's wave totals
        static_assert(3 * NP + 2 <= 4 * NP, "the sort fits the pointer-jumping area");
        int slot[PL], pp[PL];
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            pp[k] = NP;
            slot[k] = 0;
            if (i < nt) {
                const int p = s_jump[i];
                pp[k] = p < 0 ? NP : p;
                slot[k] = atomicAdd(&s_cnt[pp[k]], 1);
                atomicMin(&s_fc[pp[k]], i);
            }
        }
        lds_barrier();
        {                                               // bucket starts: two buckets per thread
            const int x0 = 2 * tid;
            const int c0 = x0 <= NP ? s_cnt[x0] : 0, c1 = x0 + 1 <= NP ? s_cnt[x0 + 1] : 0;
            int incl = c0 + c1;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(incl, d);
                if (lane >= d) incl += y;
            }
            if (lane == 63) s_ws[wave] = incl;
            lds_barrier();
            int before = incl - c0 - c1;
            for (int w = 0; w < wave; ++w) before += s_ws[w];
            if (x0 <= NP + 1) s_cnt[x0] = before;       // (entry NP + 1: the total)
            if (x0 + 1 <= NP + 1) s_cnt[x0 + 1] = before + c0;
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            if (i < nt) s_tmp[s_cnt[pp[k]] + slot[k]] = i;
        }
        lds_barrier();
        int b0[PL], b1[PL], rk[PL];
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            b0[k] = s_cnt[pp[k]];
            b1[k] = s_cnt[pp[k] + 1];
            rk[k] = 0;
            if (i < nt) {
                for (int x = b0[k]; x < b1[k]; ++x) rk[k] += s_tmp[x] < i ? 1 : 0;
                s_srt[b0[k] + rk[k]] = i;
            }
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            if (i < nt) {
                const int nsib = b0[k] + rk[k] + 1 < b1[k] ? s_srt[b0[k] + rk[k] + 1] : -1;
                s_na[i] = make_int2(nsib >= 0 ? nsib : (pp[k] == NP ? n : -1), pp[k] == NP ? -1 : pp[k]);
            }
        }
    } else {
    for (int i = tid; i < nt; i += NT) {                // bit i of its parent's children row; first child
        const int p = s_jump[i];
        const int pr = p < 0 ? NP : p;
        atomicOr(&s_cm[pr * WC + (i >> 5)], 1u << (i & 31));
        atomicMin(&s_fc[pr], i);
    }
    lds_barrier();
    for (int i = tid; i < nt; i += NT) {                // next sibling, else pending
        // (the parent's whole children row is read at once: no dependent
        // loads however far the next sibling is)
        const int p = s_jump[i];
        const uint32_t* r = s_cm + (p < 0 ? NP : p) * WC;
        uint32_t wv[WC];
#pragma unroll
        for (int w = 0; w < WC; w += 4) {
            const uint4 x4 = *reinterpret_cast<const uint4*>(r + w);
            wv[w] = x4.x;
            wv[w + 1] = x4.y;
            wv[w + 2] = x4.z;
            wv[w + 3] = x4.w;
        }
        int nsib = -1;
#pragma unroll
        for (int w = WC - 1; w >= 0; --w) {             // the lowest set bit above i wins
            const int lo = 32 * w;
            uint32_t x = wv[w];
            if (lo + 31 <= i) x = 0u;
            else if (lo <= i) x &= ~((2u << (i & 31)) - 1u);
            nsib = x ? lo + __builtin_ctz(x) : nsib;
        }
        s_na[i] = make_int2(nsib >= 0 ? nsib : (p < 0 ? n : -1), p);
    }
    }
    for (int i = tid; nt && i < NP; i += NT) {
        const int j = s_jump[i];
        s_gj[i] = make_int2((j & 0xffff) | ((int)s_hop[i] << 16), __float_as_int(s_lg[i]));
    }
    lds_barrier();
    // Pointer jumping, one node per thread and one barrier per round.  The
    // integer entries are updated in place: a read of another node's entry
    // sees it whole, before or after that node's update in the same round,
    // and either is a valid jump.  The log-gate sums alternate between two
    // copies, so that every round adds the same segments whatever the timing
    // and the sums come out the same in every run.
    // A round ends with one LDS-only barrier: a node with work left raises
    // flag rd % 3, and flag (rd + 1) % 3, the next round's, is cleared before
    // the barrier (no thread still reads it: all have passed the previous
    // round's barrier).
    auto round_more = [&](int rd, bool more) __attribute__((always_inline)) {
        if (tid == 0) s_more[(rd + 1) % 3] = 0;
        if (more) s_more[rd % 3] = 1;
        lds_barrier();
        return s_more[rd % 3] != 0;
    };
    if (nt) {
        int rd = 0;                                     // rounds so far, both loops
        // (1) the node after each subtree: the subtree root's next sibling,
        // else its parent's (a root-level node always has one); the link is
        // an ancestor such that no node from i up to below it has a next
        // sibling.  (2) With it, the path log-gates and depths: each node adds
        // its link's sums and jumps to the link's link.
        for (;; ++rd) {
            bool more = false;
#pragma unroll
            for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            if (i < nt) {
                const int2 a = s_na[i];
                if (a.x < 0) {
                    const int2 b = s_na[a.y];
                    s_na[i] = b.x >= 0 ? make_int2(b.x, a.y) : make_int2(-1, b.y);
                    more |= b.x < 0;
                }
            }
            if (i < NP) {
                const int2* src = s_gj + (rd & 1) * NP;
                const int2 a = src[i];
                const int j = (int)(int16_t)(a.x & 0xffff);
                int2 r = a;
                if (j >= 0) {
                    const int2 b = src[j];
                    const int jj = (int)(int16_t)(b.x & 0xffff);
                    r = make_int2((jj & 0xffff) | (((a.x >> 16) + (b.x >> 16)) << 16),
                                  __float_as_int(__int_as_float(a.y) + __int_as_float(b.y)));
                    more |= jj >= 0;
                }
                s_gj[((rd + 1) & 1) * NP + i] = r;
            }
            }
            if (!round_more(rd, more)) {
#pragma unroll
                for (int k = 0; k < PL; ++k) {
                    const int i = tid + k * NT;
                    if (i < NP) {                       // the last round's copy
                        const int2 a = s_gj[((rd + 1) & 1) * NP + i];
                        s_lg[i] = __int_as_float(a.y);
                        s_hop[i] = (int16_t)(a.x >> 16);
                    }
                }
                break;
            }
        }
        // preorder successor: the first child, else the node after; then each
        // node's distance to the list's end (list ranking)
        for (int i = tid; i < nt; i += NT) {
            const int f = s_fc[i];
            const int sc = f < NP ? f : s_na[i].x;
            s_rs[i] = make_int2(sc < n ? 1 : 0, sc);
        }
        lds_barrier();
        for (++rd;; ++rd) {
            bool more = false;
            for (int i = tid; i < nt; i += NT) {
                const int2 a = s_rs[i];
                if (a.y < n) {
                    const int2 b = s_rs[a.y];
                    s_rs[i] = make_int2(a.x + b.x, b.y);
                    more |= b.y < n;
                }
            }
            if (!round_more(rd, more)) break;
        }
        for (int i = tid; i < nt; i += NT) {            // position n - 1 - rank
            const int pi = min(max(n - 1 - s_rs[i].x, 0), n - 1);
            const int nx = s_na[i].x;
            s_perm[pi] = (uint16_t)i;
            s_last[pi] = (int16_t)((nx < n ? n - 1 - s_rs[nx].x : n) - 1);
        }
    }
    if (nt == 0) {
        if (!solver) {
            // the producer's first row: q into s0_r[0 .. 3], v into [4 .. 5]
            const int t0 = min(wave - kSolveWaves, (n + 15) / 16 - 1);
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) s0_r[cs] = __builtin_bit_cast(float4, cfrag(Qb, t0, cs));
            const uint16_t* vr = Vsl + (size_t)min(16 * t0 + ln, clast) * vo_row + 16 * lq;
            s0_r[4] = *reinterpret_cast<const float4*>(vr);
            s0_r[5] = *reinterpret_cast<const float4*>(vr + 8);
        }
        // a chain's path log-gates are prefix sums: a scan within each wave
        // (lane shifts) and the preceding waves' totals
        // (PL chunks of NT nodes, the chunks' wave sums in order)
        float x[PL];
        float* wsum = reinterpret_cast<float*>(s_big);
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            x[k] = i < NP ? s_lg[i] : 0.f;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float y = __shfl_up(x[k], d);
                if (lane >= d) x[k] += y;
            }
            if (lane == 63) wsum[k * kLargeWaves + wave] = x[k];
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            for (int w = 0; w < k * kLargeWaves + wave; ++w) x[k] += wsum[w];
            if (i < NP) {
                s_lg[i] = x[k];
                s_hop[i] = (int16_t)(i < n ? i + 1 : 0);
            }
        }
    }
    if constexpr (KLDS) {
#pragma unroll
        for (int kk = 0; kk < KI; ++kk) {
            const int u = wave + kk * kLargeWaves;
            if (u < NP / 4) *reinterpret_cast<u32x4*>(s_k + 4 * u * kD + 8 * lane) = k_r[kk];
        }
    } else if constexpr (!FUSED) {
        // S0 as bf16, row c at LDS row c, 16-byte chunks swizzled
#pragma unroll
        for (int k = 0; k < S0L; ++k) {
            const int x = tid + k * NT;
            if (x < 64 * kD / 4) {
                const int r = x >> 5, c4 = x & 31;      // row, float4 within the row
                uint2 w;
                w.x = (uint32_t)bf16_rne(s0s[k].x) | ((uint32_t)bf16_rne(s0s[k].y) << 16);
                w.y = (uint32_t)bf16_rne(s0s[k].z) | ((uint32_t)bf16_rne(s0s[k].w) << 16);
                *reinterpret_cast<uint2*>(s_s0 + row_chunk(r, c4 >> 1) + 4 * (c4 & 1)) = w;
            }
        }
    }
    lds_barrier();
    // ancestor rows from the preorder: j is a strict ancestor of r exactly when
    // pos(j) < pos(r) <= last(pos(j)), and only j < r can be one.  Each node's
    // (pos, last) is packed once into the free scratch (nodes past the tree
    // get pos 0xffff, never below a row's position); the tree's workgroups
    // share the (row, word) pairs, one pair per thread.
    const int nparts = Hv * 2, part = h * 2 + slice;
    uint32_t* pk = reinterpret_cast<uint32_t*>(s_big) + 16;   // (past the wave sums)
    for (int j = tid; j < NP; j += NT) {
        uint32_t v = 0xffffu;
        if (j < n) {
            const int pj = nt ? min(max(n - 1 - s_rs[j].x, 0), n - 1) : j;
            v = (uint32_t)pj | ((uint32_t)(uint16_t)s_last[pj] << 16);
        }
        pk[j] = v;
    }
#pragma unroll
    for (int k = 0; k < PL; ++k) {                      // (a max over each block's 16 lanes)
        const int i = tid + k * NT;
        if (nt && i < NP) {
            int m = s_last[i];
#pragma unroll
            for (int d = 8; d >= 1; d >>= 1) m = max(m, __shfl_xor(m, d));
            if ((i & 15) == 0) s_mlast[i >> 4] = m;
        }
    }
    if (slice == 0)
        for (int i = tid; i < n; i += NT) a.log_gamma[((size_t)b * Hv + h) * N + i] = s_lg[i];
    for (int r = part + nparts * tid; r < N; r += nparts * NT)   // depth: the rows' shares
        a.depth[(size_t)b * N + r] = r < n ? s_hop[r] - 1 : -1;
    auto node_at = [&](int pos) __attribute__((always_inline)) {   // position (clamped) -> node
        return min((int)s_perm[min(pos, n - 1)], n - 1);
    };
    // G and beta by position, through the scratch past the packed rows
    float* tl = reinterpret_cast<float*>(pk + NP);
    float* tb = tl + NP;
    static_assert((16 + 3 * NP) * 4 <= BIG, "position tables fit the ring area");
    if (nt)
        for (int i = tid; i < NP; i += NT) {
            const int v = node_at(i);
            tl[i] = i < n ? s_lg[v] : 0.f;
            tb[i] = i < n ? s_beta[v] : 0.f;
        }
    lds_barrier();
    for (int x = part + nparts * tid; x < N * W; x += nparts * NT) {
        const int r = x / W, w = x - r * W;
        uint32_t bits = 0u;
        if (r < n && 32 * w <= r) {
            const uint32_t pr = pk[r] & 0xffffu;
#pragma unroll
            for (int e = 0; e < 32; e += 4) {
                const uint4 q4 = *reinterpret_cast<const uint4*>(pk + 32 * w + e);
                const uint32_t q[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    bits |= ((q[k] & 0xffffu) < pr && pr <= (q[k] >> 16)) ? 1u << (e + k) : 0u;
            }
        }
        gm[x] = bits;
    }
    if (writer && tid == 0) a.status[b] = 0;
    if (nt)
        for (int i = tid; i < NP; i += NT) {
            s_lg[i] = tl[i];
            s_beta[i] = tb[i];
        }
    // One wave, row t in lane t, with no barrier between its steps:
    //  * occupancy: tile (t, s), s < t, holds an ancestor pair exactly when a
    //    position of block s has its subtree reaching row t; row t's occupied
    //    blocks are listed in ascending order;
    //  * the ring: row t takes the next HDR + 2 s_tn[t] + 1 slots, counted
    //    over all rows modulo RING; they may be written once every row whose
    //    slots they reuse has been released by all solve waves;
    //  * the producer items of row t: one for the diagonal block (without k
    //    in LDS also the right-hand sides), then one per C occupied blocks.
    // Prefix sums over the rows go through LDS (one read of all rows' words).
    // (A chain takes none of it.)
    if (wave == 0 && nt) {
        uint64_t occ = 0u;
#pragma unroll
        for (int sb = 0; sb < NB; sb += 4) {
            const int4 x4 = *reinterpret_cast<const int4*>(&s_mlast[sb]);
            const int ml[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                occ |= (sb + e < lane && lane < nblk && ml[e] >= 16 * lane) ? 1ull << (sb + e) : 0ull;
        }
        const int tn = __popcll(occ);
        if (lane < NB) {
            s_tn[lane] = tn;
            for (int k = 0; occ; ++k, occ &= occ - 1u) s_tcol[lane][k] = (uint8_t)__builtin_ctzll(occ);
        }
        const int sl = lane < nblk ? 2 * tn + 1 + HDR : 0;
        const int ni = lane < nblk ? NFIX + (tn + C - 1) / C : 0;
        // (slots and items of a row packed in one word: both totals stay
        // below 2^16)
        int* tmp = reinterpret_cast<int*>(s_big) + 16 + 3 * NP;   // (past the position tables)
        static_assert((16 + 3 * NP + 64) * 4 <= BIG, "row sums fit the ring area");
        tmp[lane] = sl | (ni << 16);
        int ex = 0;                                     // the rows before this lane's
#pragma unroll
        for (int r = 0; r < NB; r += 4) {
            const int4 x4 = *reinterpret_cast<const int4*>(&tmp[r]);
            ex += (r < lane ? x4.x : 0) + (r + 1 < lane ? x4.y : 0) + (r + 2 < lane ? x4.z : 0) +
                  (r + 3 < lane ? x4.w : 0);
        }
        const int gsl = ex & 0xffff;                    // first slot of row lane
        const int ib = ex >> 16;                        // first item of row lane
        const int target = gsl + sl - RING;             // rows starting below it must be released
        if (lane < NB) s_gslot[lane] = gsl;
        if (lane == NB - 1) s_gslot[NB] = gsl + sl;     // the total
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < NB; r += 4) {
            const int4 x4 = *reinterpret_cast<const int4*>(&s_gslot[r]);
            cnt += (r < lane && x4.x < target ? 1 : 0) + (r + 1 < lane && x4.y < target ? 1 : 0) +
                   (r + 2 < lane && x4.z < target ? 1 : 0) + (r + 3 < lane && x4.w < target ? 1 : 0);
        }
        if (lane < NB) s_rstar[lane] = cnt;
        for (int j = 0; j < ni; ++j) s_items[ib + j] = (uint16_t)(lane | (j << 8));
        if (lane == NB - 1) s_nitems = ib + ni;
    }
    if constexpr (UW < NB) {
        // (meanwhile, past 512 nodes) the slots of s_u: block row t is read
        // by the rows up to the one holding its last descendant; rows take
        // slots in order, each the lowest one whose holder's last reader has
        // passed, and a row that finds none is re-read from its U stores
        if (wave == 1 && nt) {
            const int ml = lane < NB ? s_mlast[lane] : 0;   // (row t's from lane t)
            int hold = -1;                              // lane x < UW: last reader of slot x's row
            int mine = -1;                              // lane t: row t's slot
            for (int t = 0; t < nblk; ++t) {
                const int endt = max(t, min(__builtin_amdgcn_readlane(ml, t) >> 4, nblk - 1));
                const uint64_t fr = __builtin_amdgcn_ballot_w64(lane < UW && hold < t);
                const int x = fr ? (int)__builtin_ctzll(fr) : -1;
                if (lane == x) hold = endt;
                if (lane == t) mine = x;
            }
            if (lane < NB) s_uslot[lane] = mine;
        }
    }
    lds_barrier();
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};

    // k / q fragment of node block blk, column chunk cs: lane (r, q) holds
    // row 16 blk + r (clamped), columns 32 cs + 8 q .. +7, from global
    // memory (a uniform base and a 32-bit lane offset); from LDS the same
    // lanes read the row's chunk 4 cs + q.
    auto gfrag = [&](const uint16_t* base, int blk, int cs) __attribute__((always_inline)) {
        const uint32_t row = (uint32_t)node_at(16 * blk + ln);
        const uint32_t off = row * (uint32_t)(kq_row * 2) + lane_col + 64u * cs;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              reinterpret_cast<const char*>(base) + off));
    };
    uint2* ring = s_big;                                // slot x: ring[64 x + lane]
    u32x4* ring16 = reinterpret_cast<u32x4*>(s_big);    // slots x, x + 1 (x even): ring16[32 x + lane]
    auto slot_at = [&](int x) __attribute__((always_inline)) { return x < RING ? x : x - RING; };

    // The diagonal block's D_t = (I + X_tt)^-1 and Y_tt from its Grams gK (lane
    // (j, q), element m: k_(4q+m) . k_j) and gQ (lane (i, q): k_(4q+m) . q_i),
    // with producer pr's LDS scratch: D_t in fp32, lane 4c + qd holding rows
    // 4qd .. +3 of column c; Y_tt (lane (i, q), element m: j = 4q + m, an
    // ancestor of i or i) as bf16.
    auto diag_block = [&](int t, int pr, f32x4 gK, f32x4 gQ, float (&accd)[4], s16x4& yb)
                          __attribute__((always_inline)) {
        const int pi = 16 * t + ln;
        const float lgi = s_lg[pi];
        // X_tt[i][j] at lane (j, q), element m: i = 4q + m
        float xv[4];
        {
            const int pj = 16 * t + ln;
            const int lj = s_last[pj];
            const float lgj = s_lg[pj];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int pi2 = 16 * t + 4 * lq + m;
                const bool anc = (pj < pi2) & (pi2 <= lj);
                const float x = s_beta[pi2] * __expf(fminf(s_lg[pi2] - lgj, 0.f)) * gK[m];
                xv[m] = anc ? x : 0.f;
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int pj = 16 * t + 4 * lq + m;
            const bool anc = (pj <= pi) & (pi <= (int)s_last[pj]);
            const float y = __expf(fminf(lgi - s_lg[pj], 0.f)) * gQ[m];
            yb[m] = (short)bf16_rne(anc ? y : 0.f);
        }
        // fp32 forward substitution, four lanes per column: lane 4c + qd
        // holds rows 4qd .. 4qd+3 of column c; step m reads column m of
        // X_tt (stored [col][row] by the lanes that hold it) and takes y_m
        // from its owner within the lane quad
        float* xd = &s_xd[pr][0];
        *reinterpret_cast<float4*>(&xd[ln * 16 + 4 * lq]) = make_float4(xv[0], xv[1], xv[2], xv[3]);
        const int c = lane >> 2, qd = lane & 3;
#pragma unroll
        for (int e = 0; e < 4; ++e) accd[e] = (4 * qd + e == c) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
            const float4 xc = *reinterpret_cast<const float4*>(&xd[m * 16 + 4 * qd]);
            const float ym = quad_bcast(accd[m & 3], m >> 2);
            const float xr[4] = {xc.x, xc.y, xc.z, xc.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {               // rows below m only
                const float upd = fmaf(-xr[e], ym, accd[e]);
                accd[e] = 4 * qd + e > m ? upd : accd[e];
            }
        }
    };

    // ================= chains =================
    // A chain (node i's parent is i - 1) is the gated delta rule's linear
    // recurrence, and the chunked form of it applies (page "Trees from
    // Marginals", section 3: the chunked linear recurrence): all nodes of
    // block row t descend from node 16 t - 1, so every ancestor outside the
    // row is folded into that node's state S_t, and no off-diagonal tile is
    // formed.  With E_t = G_(16t-1) (E_0 = 0, S_0 = S0):
    //   R_t = diag(beta)(V_t - diag(e^(G - E_t)) K_t S_t^T),  U_t = D_t R_t,
    //   O_t = diag(e^(G - E_t)) Q_t S_t^T + Y_tt U_t,
    //   S_(t+1) = e^(E_(t+1) - E_t) S_t + sum_(j in row t) e^(E_(t+1) - G_j) u_j k_j^T.
    // The producers form D_t and Y_tt and stage each row's operands in a
    // four-row LDS ring (q, v, k when it is not in LDS, K_t^T node-packed,
    // and per-node factors), so the solve waves read no global memory and
    // take no exponentials; each solve wave carries its 16 state rows in
    // fp32 as matrix-core accumulators from row to row (as the commit does)
    // and feeds their bf16 rounding straight to the next row's products.
    // The state's key columns are taken in 16-key tiles tc = 2 w + hh (keys
    // 32 w + 8 (i / 4) + 4 hh + i % 4, i = 0 .. 15), so that lane (r, q) of
    // tiles 2w and 2w + 1 holds keys 32 w + 8 q .. +7 of row r: the S0
    // registers' layout, and as bf16 one 16x16x32 operand over a 32-key
    // window; the update pairs a tile with itself against a bf16 hi and lo
    // part (the summed indices may come in any order as long as both
    // operands agree).  Every exponent is at most 0 (G only falls along the
    // chain).
    if (nt == 0) {
        constexpr int CR = 4;                           // ring rows; row t uses entry t % CR
        // D_t (A operand) and Y_tt (B operand) at slot t, past 512 nodes at
        // slot t % DT (written once the solve waves are done with row t - DT)
        constexpr int DT = UW == NB ? NB : 2 * CR;
        auto dslot = [&](int t) __attribute__((always_inline)) { return UW == NB ? t : t % DT; };
        uint2* const dtab = s_big;
        uint2* const ytab = s_big + 64 * DT;
        // entry r: v of the slice's 64 columns ([node][column], 2 KB), then
        // per node (beta, beta e^(G - E_t), e^(G - E_t), e^(E_(t+1) - G)) and
        // e^(E_(t+1) - E_t), in 2.5 KB, in the ring area; the K^T tiles (tile
        // tc: 1 KB, lane-major, each lane's four values twice: one 16x16x32
        // operand) in s_u; q and k rows as s_k (16 x 128, swizzled), q in
        // the ring area with k in LDS, else both in s_u
        constexpr int VE = 5 * 256;                     // halfwords per entry in the ring area
        uint16_t* const vring = reinterpret_cast<uint16_t*>(s_big + 64 * 2 * DT);
        constexpr int KNE = 2 * 16 * kD;                // halfwords of an entry's K^T tiles
        constexpr int QE = KNE + (KLDS ? 0 : 2 * 16 * kD);   // halfwords per entry in s_u
        // (past 512 nodes in the ring area, after the v entries)
        uint16_t* const qring = UW == NB ? reinterpret_cast<uint16_t*>(&s_u[0][0][0]) : vring + CR * VE;
        uint16_t* const qring2 = vring + CR * VE;       // (with k in LDS)
        static_assert(2 * DT * 512 + CR * VE * 2 + (KLDS ? CR * 16 * kD * 2 : 0) + (UW == NB ? 0 : CR * QE * 2) <= BIG,
                      "chain tables and ring entries fit the ring area");
        static_assert(UW < NB || UW * kSolveWaves * 512 >= CR * QE * 2, "ring entries fit s_u");
        auto vent = [&](int r) __attribute__((always_inline)) { return vring + r * VE; };
        auto fent = [&](int r) __attribute__((always_inline)) { return reinterpret_cast<float*>(vring + r * VE + 16 * 64); };
        auto knent = [&](int r) __attribute__((always_inline)) { return qring + r * QE; };
        auto qent = [&](int r) __attribute__((always_inline)) {
            return KLDS ? qring2 + r * 16 * kD : qring + r * QE + KNE;
        };
        auto kent = [&](int r) __attribute__((always_inline)) { return qring + r * QE + KNE + 16 * kD; };
        if (!solver) {
            // producer p: rows p, p + 8, ..., each row's global operands
            // requested one row ahead
            const int p = wave - kSolveWaves;
            // selection of the keys of tile 2 w + hh from a 32-key window:
            // column c takes key 8 (c / 4) + 4 hh + c % 4
            bf16x8 sel[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sel[hh][e] = (__bf16)((8 * lq + e == 8 * (ln >> 2) + 4 * hh + (ln & 3)) ? 1.f : 0.f);
            auto diag = [&](int t, const DiagOps& o) __attribute__((always_inline)) {
                bf16x8 kt[4];
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) {
                    if constexpr (KLDS)
                        kt[cs] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s_k + row_chunk(16 * t + ln, 4 * cs + lq)));
                    else kt[cs] = o.kt[cs];
                }
                f32x4 gK = z, gQ = z;
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) {
                    gK = mfma32(kt[cs], kt[cs], gK);
                    gQ = mfma32(kt[cs], o.qt[cs], gQ);
                }
                float accd[4];
                s16x4 yb;
                diag_block(t, p, gK, gQ, accd, yb);
                const int c = lane >> 2, qd = lane & 3;
                auto put_dy = [&]() __attribute__((always_inline)) {
                    uint16_t* dd = reinterpret_cast<uint16_t*>(dtab + 64 * dslot(t));
#pragma unroll
                    for (int e = 0; e < 4; ++e) dd[a16_pos(4 * qd + e, c)] = bf16_rne(accd[e]);
                    ytab[64 * dslot(t) + lane] = __builtin_bit_cast(uint2, yb);
                };
                if constexpr (UW < NB) {
                    if (t >= DT)
#pragma unroll
                        for (int gg = 0; gg < kSolveWaves; ++gg) wait_flag_ge(&s_oready[gg], t - DT + 1);
                }
                put_dy();
                // K_t^T tiles (tile 2 w + hh: its keys by the row's nodes), exact products
                s16x4 kn[8];
#pragma unroll
                for (int w = 0; w < 4; ++w)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) kn[2 * w + hh] = to_bf16x4(mfma32(kt[w], sel[hh], z));
                // per-node factors (lanes 0 .. 15: node 16 t + lane; lane 16: the decay)
                const float E0 = t > 0 ? s_lg[16 * t - 1] : 0.f;
                const float E1 = s_lg[min(16 * t + 15, NP - 1)];
                const bool more = t + 1 < nblk;
                const float gi = s_lg[16 * t + ln], bi = s_beta[16 * t + ln];
                const float ei = __expf(gi - E0);
                const float4 fac = lane < 16 ? make_float4(bi, bi * ei, ei, more ? __expf(E1 - gi) : 0.f)
                                             : make_float4(more ? __expf(E1 - E0) : 0.f, 0.f, 0.f, 0.f);
                // entry t % CR is free once every solve wave is done with row t - CR
                const int r = t % CR;
                if (t >= CR)
#pragma unroll
                    for (int gg = 0; gg < kSolveWaves; ++gg) wait_flag_ge(&s_oready[gg], t - CR + 1);
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) {
                    *reinterpret_cast<u32x4*>(qent(r) + row_chunk(ln, 4 * cs + lq)) = __builtin_bit_cast(u32x4, o.qt[cs]);
                    if constexpr (!KLDS)
                        *reinterpret_cast<u32x4*>(kent(r) + row_chunk(ln, 4 * cs + lq)) = __builtin_bit_cast(u32x4, o.kt[cs]);
                }
#pragma unroll
                for (int tc = 0; tc < 8; ++tc)
                    *reinterpret_cast<u32x4*>(knent(r) + tc * 512 + 8 * lane) =
                        __builtin_bit_cast(u32x4, __builtin_shufflevector(kn[tc], kn[tc], 0, 1, 2, 3, 4, 5, 6, 7));
                uint16_t* vw = vent(r) + ln * 64 + 16 * lq;
                *reinterpret_cast<u32x4*>(vw) = o.vt[0];
                *reinterpret_cast<u32x4*>(vw + 8) = o.vt[1];
                if (lane <= 16) reinterpret_cast<float4*>(fent(r))[lane] = fac;
                publish_set(&s_done[t], 1, lane);
            };
            DiagOps da, db;                             // (row p's q and v: requested in the setup)
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
                da.qt[cs] = __builtin_bit_cast(bf16x8, s0_r[cs]);
                if constexpr (!KLDS) da.kt[cs] = cfrag(Kb, p, cs);
            }
            da.vt[0] = __builtin_bit_cast(u32x4, s0_r[4]);
            da.vt[1] = __builtin_bit_cast(u32x4, s0_r[5]);
            for (int t = p; t < nblk; t += 2 * kProducers) {
                dfetch(t + kProducers, db);
                diag(t, da);
                if (t + kProducers >= nblk) break;
                dfetch(t + 2 * kProducers, da);
                diag(t + kProducers, db);
            }
            return;
        }
        __builtin_amdgcn_s_setprio(2);
        const int g = wave;
        const int c0 = cbase + 16 * g;
        // the wave's state rows: lane (r, q) of tile 2 w + hh holds row
        // c0 + r, keys 32 w + 8 q + 4 hh .. +3 (S0's as requested before the
        // setup; fused: the rows this wave committed, re-read after a fence
        // that orders its own stores before the loads)
        f32x4 st[8];
        if constexpr (FUSED || !KLDS) {
            if constexpr (FUSED) __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            const float* Sp = (FUSED ? c.S_out : a.S0) + ((size_t)b * Hv + h) * kD * kD + (size_t)(c0 + ln) * kD + 8 * lq;
#pragma unroll
            for (int tc = 0; tc < 8; ++tc) st[tc] = *reinterpret_cast<const f32x4*>(Sp + 32 * (tc >> 1) + 4 * (tc & 1));
        } else {
#pragma unroll
            for (int tc = 0; tc < 8; ++tc) st[tc] = __builtin_bit_cast(f32x4, s0_r[tc]);
        }
        s16x4 ident;
#pragma unroll
        for (int e = 0; e < 4; ++e) ident[e] = (4 * lq + e == ln) ? (short)0x3f80 : (short)0;
        const __amdgpu_buffer_rsrc_t u_rsrc =
            __builtin_amdgcn_make_buffer_rsrc(Ug, (short)0, N * kD * 4, kBufferFlags);
        const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            O + vo_base, (short)0, ((n - 1) * Hv + 1) * kD * 2, kBufferFlags);
        // keys 32 w + 8 q .. +7 of row r of a 16 x 128 block swizzled as s_k
        auto win = [&](const uint16_t* blk, int r, int w) __attribute__((always_inline)) {
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(blk + row_chunk(r, 4 * w + lq)));
        };
        // two 4-index halves as one 16x16x32 operand
        auto cat = [](s16x4 x, s16x4 y) __attribute__((always_inline)) {
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // K_t S_t^T: [node 4q + m][column], from the row's k rows in LDS
        // (s_k itself, or the ring entry) and the state's bf16 rounding sb
        s16x4 sb[8];
        f32x4 ks;
        auto kst = [&](const uint16_t* kb) __attribute__((always_inline)) {
            f32x4 k1 = z, k2 = z;
#pragma unroll
            for (int w = 0; w < 4; w += 2) {
                k1 = mfma32(win(kb, ln, w), cat(sb[2 * w], sb[2 * w + 1]), k1);
                k2 = mfma32(win(kb, ln, w + 1), cat(sb[2 * w + 2], sb[2 * w + 3]), k2);
            }
            return k1 + k2;
        };
#pragma unroll
        for (int tc = 0; tc < 8; ++tc) sb[tc] = to_bf16x4(st[tc]);
        if constexpr (KLDS) ks = kst(s_k);
        // Row t.  With k in LDS the next row's K S^T is formed in the same
        // step as this row's outputs.  Each row's flag is read during the row
        // before (its latency under that row's stores) and waited on only
        // when it was not yet set.
        int fl = __hip_atomic_load(&s_done[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        for (int t = 0; t < nblk; ++t) {
            const int pr = 16 * t + ln;
            const int r = t % CR;
            if (__builtin_amdgcn_readfirstlane(fl) < 1) wait_flag_ge(&s_done[t], 1);
            asm volatile("" ::: "memory");
            if constexpr (!KLDS) ks = kst(kent(r));
            const float4* fr = reinterpret_cast<const float4*>(fent(r));
            float4 fn[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) fn[m] = fr[4 * lq + m];
            const float eo = fr[ln].z, dec = fr[16].x;
            const s16x4 vt = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2*>(vent(r) + ln * 64 + 16 * g + 4 * lq));
            const f32x4 vd = mfma16(vt, ident, z);
            f32x4 acc;
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = fn[m].x * vd[m] - fn[m].y * ks[m];
            const s16x4 dt = __builtin_bit_cast(s16x4, dtab[64 * dslot(t) + lane]);
            const s16x4 ytt = __builtin_bit_cast(s16x4, ytab[64 * dslot(t) + lane]);
            s16x4 hi, lo;
            split4(acc, hi, lo);
            const f32x4 uf = mfma32(cat(dt, dt), cat(hi, lo), z);   // lane (c, q): nodes 4q + m, column c
            const s16x4 ut = to_bf16x4(uf);
            // the next row's state (the chain every row waits for; after
            // the last row the factors are 0 and it is not used)
            {
                f32x4 wu;
#pragma unroll
                for (int m = 0; m < 4; ++m) wu[m] = fn[m].w * uf[m];
                s16x4 wh, wl;
                split4(wu, wh, wl);
                const uint16_t* knb = knent(r) + 8 * lane;
#pragma unroll
                for (int tc = 0; tc < 8; ++tc) {
                    const bf16x8 kn = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(knb + tc * 512));
                    st[tc] = mfma32(kn, cat(wh, wl), st[tc] * dec);
                }
            }
            // e^(G - E_t) Q_t S_t^T + Y_tt U_t: [column 4q + m][node]
            const uint16_t* qb = qent(r);
            f32x4 oc = z, oc2 = z;
#pragma unroll
            for (int w = 0; w < 4; w += 2) {
                oc = mfma32(cat(sb[2 * w], sb[2 * w + 1]), win(qb, ln, w), oc);
                oc2 = mfma32(cat(sb[2 * w + 2], sb[2 * w + 3]), win(qb, ln, w + 1), oc2);
            }
#pragma unroll
            for (int tc = 0; tc < 8; ++tc) sb[tc] = to_bf16x4(st[tc]);
            if constexpr (KLDS) ks = kst(s_k + 16 * min(t + 1, nblk - 1) * kD);
            oc = (oc + oc2) * eo;
            oc = mfma16(ut, ytt, oc);
            publish_set(&s_oready[g], t + 1, lane);     // the row's ring entry is read
            fl = __hip_atomic_load(&s_done[min(t + 1, nblk - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            // the cache rows (lane (n, q): nodes 4q .. 4q+3 of column n) and
            // outputs; positions past the tree store outside the buffers
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                const int i = 16 * t + 4 * lq + mm;
                const int off = i < n ? (i * kD + c0 + ln) * 4 : 0x7fffffff;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(uf[mm]), u_rsrc, off, 0, 0);
            }
            const int orow = pr < n ? (pr * Hv * kD + c0 + 4 * lq) * 2 : 0x7fffffff;
            const s16x4 ob = to_bf16x4(oc);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ob), o_rsrc, orow, 0, 0);
        }
        return;
    }

    if (solver) {
        // ================= solve waves =================
        // (the solve is the chain every row waits for: its waves issue ahead
        // of the producers sharing their SIMDs)
        __builtin_amdgcn_s_setprio(2);
        const int g = wave;
        const int c0 = cbase + 16 * g;                  // this wave's first value column
        // with k in LDS, s0g: this wave's 16 S0 rows as bf16, lane (r, q)
        // holding row c0 + r, columns 32 cs + 8 q .. +7; the A operand S0 (for
        // S0 Q^T) and the B operand S0^T (for K S0^T)
        s16x4 ident;
#pragma unroll
        for (int e = 0; e < 4; ++e) ident[e] = (4 * lq + e == ln) ? (short)0x3f80 : (short)0;
        const __amdgpu_buffer_rsrc_t u_rsrc =
            __builtin_amdgcn_make_buffer_rsrc(Ug, (short)0, N * kD * 4, kBufferFlags);
        const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            O + vo_base, (short)0, ((n - 1) * Hv + 1) * kD * 2, kBufferFlags);
        const char* Vb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.v) + vo_base + c0 + 4 * lq);
        // with k in LDS, a row's global operands, requested one row ahead: q,
        // and v of this wave's columns (lane (r, q): row r, columns 4 q .. +3).
        // Without, the producers form the row's right-hand sides.
        struct RowOps {
            bf16x8 qt[4];
            uint2 vt;
        };
        auto fetch = [&](int t, RowOps& r) __attribute__((always_inline)) {
            t = min(t, nblk - 1);
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) r.qt[cs] = gfrag(Qb, t, cs);
            const uint32_t vr = (uint32_t)node_at(16 * t + ln) * (uint32_t)(vo_row * 2);
            r.vt = *reinterpret_cast<const uint2*>(Vb + vr);
        };
        // One row: every LDS operand that does not wait for the producers is
        // requested first (the row's blocks, node indices, gates, this wave's
        // own U rows of the first SB occupied blocks), then the right-hand
        // side and e^G Q S0^T are formed, then the wait, then the row's tiles.
        // The first SB occupied blocks' operands are read together, the
        // unused ones skipped by uniform branches; rows with more take a loop.
        constexpr int SB = 8;
        constexpr int TW = NB / 4;                      // words of a row of s_tcol
        // U_sb as the B operand of row t (sb = t: an unused entry): from LDS
        // when kept there; past 512 nodes a row without a slot is re-read
        // from this lane's own fp32 stores of it (rows 4q .. 4q+3 of column
        // c0 + n, past L1), rounded as LDS keeps it, and positions past the
        // tree read as zero
        const int slotv = UW < NB && lane < NB ? s_uslot[min(lane, NB - 1)] : -1;   // lane t: row t's slot
        auto uget = [&](int sb, int t) __attribute__((always_inline)) {
            if constexpr (UW == NB) {
                return __builtin_bit_cast(s16x4, s_u[sb][g][lane]);
            } else {
                const int us = __builtin_amdgcn_readlane(slotv, sb);
                if (us >= 0 || sb == t) return __builtin_bit_cast(s16x4, s_u[max(us, 0)][g][lane]);
                f32x4 x;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int i = 16 * sb + 4 * lq + m;
                    const int off = (node_at(i) * kD + c0 + ln) * 4;
                    const float y = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(u_rsrc, off, 0, 1));
                    x[m] = i < n ? y : 0.f;
                }
                return to_bf16x4(x);
            }
        };
        auto row = [&](int t, RowOps& r) __attribute__((always_inline)) {
            const int nts = __builtin_amdgcn_readfirstlane(s_tn[t]);
            const int base = __builtin_amdgcn_readfirstlane(s_gslot[t]) % RING;
            uint32_t tw[TW];
#pragma unroll
            for (int w = 0; w < TW; ++w)
                tw[w] = __builtin_amdgcn_readfirstlane(reinterpret_cast<const uint32_t*>(&s_tcol[t][0])[w]);
            const int pr = 16 * t + ln;                 // this lane's node of the products' columns
            const int no = node_at(pr);
            int nu[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) nu[m] = node_at(16 * t + 4 * lq + m);
            s16x4 ub[SB], xa[SB], ya[SB];
#pragma unroll
            for (int e = 0; e < SB; ++e) {
                const int sb = e < nts ? (int)((tw[e >> 2] >> (8 * (e & 3))) & 0xffu) : t;
                ub[e] = uget(sb, t);
            }
            f32x4 acc, oc;
            if constexpr (KLDS) {
                // R_t = diag(beta)(V_t - diag(e^G) K_t S0^T): [node 4q + m][column]
                // (V moves into the accumulator layout by an exact product with I)
                float bt[4], lgr[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    bt[m] = s_beta[16 * t + 4 * lq + m];
                    lgr[m] = s_lg[16 * t + 4 * lq + m];
                }
                const float lgc = s_lg[pr];
                f32x4 ks = z;
#pragma unroll
                for (int cs = 0; cs < 4; ++cs)
                    ks = mfma32(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s_k + row_chunk(no, 4 * cs + lq))),
                                s0g[cs], ks);
                const f32x4 vd = mfma16(__builtin_bit_cast(s16x4, r.vt), ident, z);
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[m] = bt[m] * (vd[m] - __expf(lgr[m]) * ks[m]);
                // e^G Q_t S0^T: [column 4q + m][node]
                oc = z;
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) oc = mfma32(s0g[cs], r.qt[cs], oc);
                oc *= __expf(lgc);
            }
            wait_flag_ge(&s_done[t], nts + NFIX);
            if constexpr (!KLDS) {                      // the producers' right-hand sides
                acc = __builtin_bit_cast(f32x4, ring16[slot_at(base + 2 * g) * 32 + lane]);
                oc = __builtin_bit_cast(f32x4, ring16[slot_at(base + 8 + 2 * g) * 32 + lane]);
            }
            // U_t = D_t (R_t - sum_s X_ts U_s) (the slots hold -X) and
            // O_t += sum_{s < t} Y_ts U_s as U^T Y^T; a row's Y tiles follow
            // its -X tiles, the diagonal block's last
            const int xb = base + HDR;
#pragma unroll
            for (int e = 0; e < SB; ++e) {
                xa[e] = __builtin_bit_cast(s16x4, ring[slot_at(xb + e) * 64 + lane]);
                ya[e] = __builtin_bit_cast(s16x4, ring[slot_at(xb + nts + e) * 64 + lane]);
            }
            s16x4 dt;
            if constexpr (KLDS) dt = __builtin_bit_cast(s16x4, s_d[t][lane]);
            else dt = __builtin_bit_cast(s16x4, ring[slot_at(base + 16) * 64 + lane]);
            const s16x4 ytt = __builtin_bit_cast(s16x4, ring[slot_at(xb + 2 * nts) * 64 + lane]);
            f32x4 acc2 = z, oc2 = z;
#pragma unroll
            for (int e = 0; e < SB; ++e) {
                // (a uniform branch skips an unused entry, whose LDS may hold
                // any bits, NaN included)
                if (e < nts) {
                    if (e & 1) {
                        acc2 = mfma16(xa[e], ub[e], acc2);
                        oc2 = mfma16(ub[e], ya[e], oc2);
                    } else {
                        acc = mfma16(xa[e], ub[e], acc);
                        oc = mfma16(ub[e], ya[e], oc);
                    }
                }
            }
            for (int m0 = SB; m0 < nts; m0 += SB) {
#pragma unroll
                for (int e = 0; e < SB; ++e) {
                    const int m = m0 + e;
                    const int sb = m < nts ? __builtin_amdgcn_readfirstlane((int)s_tcol[t][m]) : t;
                    ub[e] = uget(sb, t);
                    xa[e] = __builtin_bit_cast(s16x4, ring[slot_at(xb + m) * 64 + lane]);
                    ya[e] = __builtin_bit_cast(s16x4, ring[slot_at(xb + nts + m) * 64 + lane]);
                }
#pragma unroll
                for (int e = 0; e < SB; ++e)
                    if (m0 + e < nts) {
                        if (e & 1) {
                            acc2 = mfma16(xa[e], ub[e], acc2);
                            oc2 = mfma16(ub[e], ya[e], oc2);
                        } else {
                            acc = mfma16(xa[e], ub[e], acc);
                            oc = mfma16(ub[e], ya[e], oc);
                        }
                    }
            }
            acc += acc2;
            s16x4 hi, lo;                               // (bf16 hi + lo parts: D_t meets R to ~16 bits)
            split4(acc, hi, lo);
            const f32x4 uf = mfma16(dt, lo, mfma16(dt, hi, z));
            const s16x4 ut = to_bf16x4(uf);
            if constexpr (UW == NB) {
                s_u[t][g][lane] = __builtin_bit_cast(uint2, ut);
            } else {
                const int x = __builtin_amdgcn_readlane(slotv, t);
                if (x >= 0) s_u[x][g][lane] = __builtin_bit_cast(uint2, ut);
            }
            // the cache row: lane (n, q) holds rows 4q .. 4q+3 of column n;
            // positions past the tree store outside the buffer and are dropped
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                const int i = 16 * t + 4 * lq + mm;
                const int off = i < n ? (nu[mm] * kD + c0 + ln) * 4 : 0x7fffffff;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(uf[mm]), u_rsrc, off, 0, 0);
            }
            oc += oc2;
            oc = mfma16(ut, ytt, oc);                   // the diagonal block
            publish_set(&s_oready[g], t + 1, lane);     // the row's slots are read: release them
            const int orow = pr < n ? (no * Hv * kD + c0 + 4 * lq) * 2 : 0x7fffffff;
            u32x2 w;
            w[0] = (uint32_t)bf16_rne(oc[0]) | ((uint32_t)bf16_rne(oc[1]) << 16);
            w[1] = (uint32_t)bf16_rne(oc[2]) | ((uint32_t)bf16_rne(oc[3]) << 16);
            __builtin_amdgcn_raw_buffer_store_b64(w, o_rsrc, orow, 0, 0);
        };
        RowOps ra, rb;
        if constexpr (KLDS) {
            fetch(0, ra);
            // Nothing of the setup is in flight past this point but the first
            // row's operands, so the loop's waits count only its own requests.
            wait_vmem_le<5>();
            if constexpr (!FUSED) {
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) s0g[cs] = to_bf16x8(s0_r[2 * cs], s0_r[2 * cs + 1]);
            }
            for (int t = 0; t < nblk; t += 2) {
                fetch(t + 1, rb);
                row(t, ra);
                if (t + 1 >= nblk) break;
                fetch(t + 2, ra);
                row(t + 1, rb);
            }
        } else {
            wait_vmem_all();
            for (int t = 0; t < nblk; ++t) row(t, ra);
        }
        return;
    }

    // ================= producers =================
    const int p = wave - kSolveWaves;                   // 0 .. kProducers - 1
    const int nitems = s_nitems;
    const uint16_t* Vs = static_cast<const uint16_t*>(a.v) + vo_base + cbase;   // v of the slice's columns
    // An item's operands, requested during the previous item: its row, that row's
    // slots and occupied blocks, the node rows of its k fragments, q of its
    // row and, when k is not in LDS, k of its row and either k of its
    // column block (C = 1) or, for the diagonal item, v of its row
    // (the slice's 64 columns in two 32-column windows: lane (r, q) holds
    // row r, columns 32 w + 8 q .. +7 of window w, in the same registers).
    struct ItemOps {
        int t, j, nts, base;
        int sb[C];                                      // the item's column blocks (t: none)
        int rt, rx[C];                                  // k rows (nodes) of lane ln in the row's / blocks' fragments
        bf16x8 kt[KLDS ? 1 : 4];
        u32x4 kx[KLDS ? 1 : C][KLDS ? 1 : 4];
        bf16x8 qt[4];
    };
    static_assert(KLDS || C == 1, "v shares the registers of one column block's k");
    auto fetch = [&](int it, ItemOps& o) __attribute__((always_inline)) {
        const int code = __builtin_amdgcn_readfirstlane((int)s_items[min(it, nitems - 1)]);
        const int t = code & 0xff, j = code >> 8;
        o.t = t;
        o.j = j;
        o.nts = __builtin_amdgcn_readfirstlane(s_tn[t]);
        o.base = __builtin_amdgcn_readfirstlane(s_gslot[t]) % RING;
        o.rt = node_at(16 * t + ln);
#pragma unroll
        for (int e = 0; e < C; ++e) {
            const int m = (j - NFIX) * C + e;
            o.sb[e] = j >= NFIX && m < o.nts ? __builtin_amdgcn_readfirstlane((int)s_tcol[t][m]) : t;
            o.rx[e] = node_at(16 * o.sb[e] + ln);
        }
        const uint32_t qoff = (uint32_t)o.rt * (uint32_t)(kq_row * 2) + lane_col;
#pragma unroll
        for (int cs = 0; cs < 4; ++cs)
            o.qt[cs] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                      reinterpret_cast<const char*>(Qb) + qoff + 64u * cs));
        if constexpr (!KLDS) {
#pragma unroll
            for (int cs = 0; cs < 4; ++cs)
                o.kt[cs] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                          reinterpret_cast<const char*>(Kb) + qoff + 64u * cs));
            // (the same four requests for either: a branch here would make
            // the compiler join two register sets, waiting for their loads)
            const char* pk = reinterpret_cast<const char*>(Kb) + (uint32_t)o.rx[0] * (uint32_t)(kq_row * 2) + lane_col;
            const char* pv = reinterpret_cast<const char*>(Vs) + (uint32_t)o.rt * (uint32_t)(vo_row * 2) + lane_col;
            const bool isv = j == 0;
#pragma unroll
            for (int cs = 0; cs < 4; ++cs)
                o.kx[0][cs] = *reinterpret_cast<const u32x4*>(isv ? pv + 64 * (cs & 1) : pk + 64 * cs);
        }
    };
    auto wait_ring = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int gg = 0; gg < kSolveWaves; ++gg) wait_flag_ge(&s_oready[gg], s_rstar[t]);
    };
    // One item: its products from o, then o is refilled with the item nxt's
    // operands (so their requests overlap this item's remaining work: masks,
    // substitution, the ring wait and stores), then the rest.
    auto work = [&](ItemOps& o, int nxt) __attribute__((always_inline)) {
        const int t = o.t, j = o.j, nts = o.nts, base = o.base;
        int sb[C];
#pragma unroll
        for (int e = 0; e < C; ++e) sb[e] = o.sb[e];
        const int pi = 16 * t + ln;                     // the Gram columns' node i
        const float lgi = s_lg[pi];
        // (without k in LDS the diagonal item also forms the row's right-hand sides)
        const bool diag = j == 0;
        // ---- products ----
        f32x4 gA[C], gB[C];    // diagonal item: X_tt, Y_tt Grams; else -X_ts, Y_ts Grams of its blocks
        {
            bf16x8 kt[4];
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
                if constexpr (KLDS)
                    kt[cs] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s_k + row_chunk(o.rt, 4 * cs + lq)));
                else kt[cs] = o.kt[cs];
            }
#pragma unroll
            for (int e = 0; e < C; ++e) gA[e] = gB[e] = z;
            if (diag) {
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) {
                    gA[0] = mfma32(kt[cs], kt[cs], gA[0]);     // lane (j, q): k_{4q+m} . k_j
                    gB[0] = mfma32(kt[cs], o.qt[cs], gB[0]);   // lane (i, q): k_{4q+m} . q_i
                }
                if constexpr (!KLDS) {
                    // ---- the row's right-hand sides, for the four column groups ----
                    wait_ring(t);
                    float bt[4], eg[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        bt[m] = s_beta[16 * t + 4 * lq + m];
                        eg[m] = __expf(s_lg[16 * t + 4 * lq + m]);
                    }
                    const float egc = __expf(lgi);
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {
                        // R_t = diag(beta)(V_t - diag(e^G) K_t S0^T): [node 4q + m][column];
                        // e^G Q_t S0^T: [column 4q + m][node]
                        f32x4 ks = z, pc = z;
#pragma unroll
                        for (int cs = 0; cs < 4; ++cs) {
                            const bf16x8 sf = __builtin_bit_cast(
                                bf16x8, *reinterpret_cast<const u32x4*>(s_s0 + row_chunk(16 * gg + ln, 4 * cs + lq)));
                            ks = mfma32(kt[cs], sf, ks);
                            pc = mfma32(sf, o.qt[cs], pc);
                        }
                        // V of the group into the accumulator layout: an exact
                        // product of its window with the columns 16 (gg % 2) ..
                        // +15 of a 32 x 16 selection
                        bf16x8 sel;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            sel[e] = (__bf16)((8 * lq + e == 16 * (gg & 1) + ln) ? 1.f : 0.f);
                        const f32x4 vd = mfma32(__builtin_bit_cast(bf16x8, o.kx[0][gg >> 1]), sel, z);
                        f32x4 R;
#pragma unroll
                        for (int m = 0; m < 4; ++m) R[m] = bt[m] * (vd[m] - eg[m] * ks[m]);
                        pc *= egc;
                        ring16[slot_at(base + 2 * gg) * 32 + lane] = __builtin_bit_cast(u32x4, R);
                        ring16[slot_at(base + 8 + 2 * gg) * 32 + lane] = __builtin_bit_cast(u32x4, pc);
                    }
                }
            } else {
#pragma unroll
                for (int cs = 0; cs < 4; ++cs)
#pragma unroll
                    for (int e = 0; e < C; ++e) {
                        bf16x8 kx;
                        if constexpr (KLDS)
                            kx = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s_k + row_chunk(o.rx[e], 4 * cs + lq)));
                        else kx = __builtin_bit_cast(bf16x8, o.kx[e][cs]);
                        gA[e] = mfma32(kx, kt[cs], gA[e]);     // lane (i, q): k_{j = 4q+m} . k_i
                        gB[e] = mfma32(kx, o.qt[cs], gB[e]);   // lane (i, q): k_j . q_i
                    }
            }
        }
        fetch(nxt, o);
        int done = 1;
        if (diag) {
            // ---- D_t = (I + X_tt)^-1 and Y_tt ----
            float accd[4];
            s16x4 yb;
            diag_block(t, p, gA[0], gB[0], accd, yb);
            const int c = lane >> 2, qd = lane & 3;
            uint16_t* dd = KLDS ? reinterpret_cast<uint16_t*>(&s_d[t][0])
                                : reinterpret_cast<uint16_t*>(&ring[slot_at(base + 16) * 64]);
            wait_ring(t);
#pragma unroll
            for (int e = 0; e < 4; ++e) dd[a16_pos(4 * qd + e, c)] = bf16_rne(accd[e]);
            ring[slot_at(base + HDR + 2 * nts) * 64 + lane] = __builtin_bit_cast(uint2, yb);
        } else {
            // ---- -X_ts and Y_ts for C occupied blocks s ----
            const float bi = s_beta[pi];
            s16x4 xn[C], yv[C];
#pragma unroll
            for (int e = 0; e < C; ++e)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int pj = 16 * sb[e] + 4 * lq + m;
                    const bool anc = pi <= (int)s_last[pj];      // (pj < pi: s < t)
                    const float dec = __expf(fminf(lgi - s_lg[pj], 0.f));
                    xn[e][m] = (short)bf16_rne(anc ? -bi * dec * gA[e][m] : 0.f);
                    yv[e][m] = (short)bf16_rne(anc ? dec * gB[e][m] : 0.f);
                }
            wait_ring(t);
            done = 0;
#pragma unroll
            for (int e = 0; e < C; ++e) {
                const int mm = (j - NFIX) * C + e;
                if (mm < nts) {
                    ring[slot_at(base + HDR + mm) * 64 + lane] = __builtin_bit_cast(uint2, xn[e]);
                    ring[slot_at(base + HDR + nts + mm) * 64 + lane] = __builtin_bit_cast(uint2, yv[e]);
                    ++done;
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane == 0) __hip_atomic_fetch_add(&s_done[t], done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    ItemOps io;
    fetch(p, io);
    // (as for the solve waves: only the first item's operands are in flight)
    wait_vmem_le<KLDS ? 4 : 4 + 4 + 4>();
    // Items after each producer's first are claimed in list order from an LDS
    // counter, one item ahead, so that a producer done early takes the next.
    for (int it = p; it < nitems;) {
        int nxt = 0;
        if (lane == 0) nxt = __hip_atomic_fetch_add(&s_claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        nxt = __builtin_amdgcn_readfirstlane(nxt) + kProducers;
        work(io, nxt);
        it = nxt;
    }
}

}  // namespace

bool verify_large_supported(const VerifyArgs& a, int io) {
    return io == GDN_BF16 && a.dk == kD && a.dv == kD && a.N > 128 && a.N <= kLargeMaxN;
}

namespace {

hipError_t launch_large(const VerifyArgs& a, const CommitArgs* c, hipStream_t stream) {
    VerifyArgs copy = a;
    CommitArgs ccopy{};
    if (c) ccopy = *c;
    // two 64-column slices per (sequence, value head); a unit's slices are
    // 8 workgroups apart, so both run on one XCD
    int units = a.B * a.Hv;
    const unsigned grid = 16u * (unsigned)((units + 7) / 8);
    const void* fn = a.N <= 256   ? (c ? (const void*)verify_large_kernel<16, true> : (const void*)verify_large_kernel<16, false>)
                     : a.N <= 512 ? (c ? (const void*)verify_large_kernel<32, true> : (const void*)verify_large_kernel<32, false>)
                                  : (c ? (const void*)verify_large_kernel<64, true> : (const void*)verify_large_kernel<64, false>);
    void* args[] = {&copy, &ccopy, &units};
    return hipLaunchKernel(fn, dim3(grid), dim3(kLargeThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_verify_large(const VerifyArgs& a, int io, hipStream_t stream) {
    (void)io;
    return launch_large(a, nullptr, stream);
}

hipError_t launch_commit_verify_large(const VerifyArgs& a, const CommitArgs& c, int io, hipStream_t stream) {
    (void)io;
    return launch_large(a, &c, stream);
}

}  // namespace gdn
