// verify_large.hip -- MFMA tree verification for d_k = d_v = 128, bf16
// q/k/v/o and trees of 129 .. 16 * NB nodes (NB = 16 or 32 blocks of 16 nodes).
//
// Same method as the small-tree kernel (page "Trees from Marginals:
// Autoregressive drafting with factorized priors", section 3: the Gram matrix,
// a tiled forward substitution and the output stage, fused), laid out for
// trees whose interaction tiles do not fit in LDS.  One workgroup per
// (sequence, value head, 64-column slice), twelve waves in two roles that
// meet through LDS flags, with no barrier after the setup:
//
//  * setup (all waves): the parent row is checked, the tree's nodes are
//    relabelled in preorder (every subtree one run of positions, so ancestry
//    is an interval test and a block row's ancestors sit in few column
//    blocks), the path log-gates are summed by pointer doubling, and the
//    tree's workgroups share writing its ancestor rows, depths and status.
//    The workgroup's global inputs are requested first (for trees of up to
//    256 nodes the k rows, stored into LDS at its end), so their latency
//    overlaps it; its barriers order LDS only.
//  * row owners (waves 4 .. 11, 16-position block rows round robin): for a
//    row t, the diagonal block's inverse D_t = (I + X_tt)^-1 (fp32, kept bf16),
//    every occupied tile of the row already multiplied by it,
//    X~_ts = D_t X_ts, and the right-hand side D_t R_t with
//    R_t = diag(beta)(V_t - diag(e^G) K_t S0^T) (bf16 hi + lo parts of R),
//    into a ring of LDS slots.  With those the substitution of a row is
//    U_t = D_t R_t - sum_s X~_ts U_s: one chain of 16x16x16 products, the last
//    of which waits for the previous row.  Then the row's outputs
//    O_t = e^G Q_t S0^T + sum_{s <= t} Y_ts U_s, with the Y tiles formed from
//    the same k operands and U read from LDS as the solve publishes it.
//  * solve (waves 0 .. 3, 16 value columns each): row by row, the chain of
//    the row's X~ products on D_t R_t; U_t goes to LDS (bf16, for later rows
//    and the outputs) and to the cache (fp32).  The solve waves read no
//    global memory.
//
// Inputs are gathered and outputs written at the caller's node indices.
#include "gdn_common.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"

namespace gdn {

namespace {

constexpr int kLargeMaxN = 512;      // largest tree of this path
constexpr int kLargeWaves = 12;
constexpr int kLargeThreads = 64 * kLargeWaves;
constexpr int kSolveWaves = 4;       // one 16-column group each: 64 columns per workgroup
constexpr int kOwners = kLargeWaves - kSolveWaves;
constexpr int kChunkG = 3;           // k operands of a row's tiles requested together (global memory)
constexpr int kChunkL = 2;           // ... read together (LDS)

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
    static constexpr int WC = NP / 32;                  // words of a children row
    static constexpr int SCRATCH = ((NP + 1) * WC + 5 * NP + 1) * 4;   // the preorder's
    static constexpr int RING0 = NB <= 16 ? 84 * 512 : 136 * 512;
    static constexpr int BIG = RING0 > SCRATCH ? RING0 : SCRATCH;
    static constexpr int RING = BIG / 1024 * 2;         // 512-byte slots in flight (even)
};

template <int NB>
__global__ __launch_bounds__(kLargeThreads, 1) void verify_large_kernel(VerifyArgs a, int units) {
    using L = LargeShape<NB>;
    constexpr int kChunk = L::KLDS ? kChunkL : kChunkG;
    constexpr int NP = L::NP;
    constexpr int NT = kLargeThreads;
    constexpr bool KLDS = L::KLDS;
    constexpr int WC = L::WC;
    constexpr int SCRATCH = L::SCRATCH;
    constexpr int BIG = L::BIG;
    constexpr int RING = L::RING;
    constexpr int PL = (NP + NT - 1) / NT;              // tree entries per thread
    // the ring: per row, D_t R_t of the four column groups (two slots each,
    // 16 bytes per lane) and the row's -X~ tiles (8 bytes per lane each);
    // during the setup the preorder's scratch
    __shared__ __attribute__((aligned(16))) uint2 s_big[BIG / 8];
    __shared__ __attribute__((aligned(16))) uint16_t s_k[KLDS ? NP * kD : 8];   // k rows, node order
    __shared__ __attribute__((aligned(16))) uint16_t s_s0[64 * kD];            // the slice's S0 rows, bf16
    __shared__ __attribute__((aligned(16))) uint2 s_u[NB][kSolveWaves][64];   // U_t, bf16 B operands
    __shared__ __attribute__((aligned(16))) float s_lg[NP];
    __shared__ __attribute__((aligned(16))) float s_beta[NP];
    __shared__ __attribute__((aligned(16))) int32_t s_jump[NP];
    __shared__ uint16_t s_perm[NP];                     // position -> node
    __shared__ __attribute__((aligned(8))) int16_t s_last[NP];   // position of the last descendant
    __shared__ int16_t s_hop[NP];                       // nodes on the path to the root (depth + 1)
    __shared__ int s_mlast[NB];                         // largest s_last of each block
    __shared__ uint8_t s_tcol[NB][NB];                  // row t's occupied blocks s < t, ascending
    __shared__ int s_tn[NB];                            // their number
    __shared__ int s_gslot[NB + 1];                     // first tile of row t, counted over all rows
    __shared__ int s_rstar[NB];                         // rows consumed before row t's ring slots are free
    __shared__ int s_xready[NB];                        // row t's ring slots published
    __shared__ int s_uready[kSolveWaves];               // rows finished by each solve wave
    __shared__ int s_more[9];                           // per-round flags of the three doubling loops
    __shared__ int s_bad;                               // first node with an invalid parent
    __shared__ int s_notchain;                          // some node's parent is not the node before it

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
    // the slice's 64 S0 rows (fp32; converted into LDS after the setup)
    constexpr int S0L = 64 * kD / 4 / NT + 1;           // float4 loads per thread
    float4 s0_r[S0L];
    const float* S0p = a.S0 + ((size_t)b * Hv + h) * kD * kD + (size_t)cbase * kD;
#pragma unroll
    for (int k = 0; k < S0L; ++k) {                     // (float4 index in the 64 x 128 slice, clamped)
        const int x = min(tid + k * NT, 64 * kD / 4 - 1);
        s0_r[k] = *reinterpret_cast<const float4*>(S0p + 4 * x);
    }
    // k rows of the tree (node order, rows past the tree copy row n - 1) into
    // registers, written to LDS at the end of the setup: one 1 KB unit is
    // four rows, lane l taking row 4u + l / 16 and its logical chunk
    // (l % 16) ^ (row & 15), so the store is one contiguous 16-byte write per lane
    constexpr int KI = KLDS ? (NP / 4 + kLargeWaves - 1) / kLargeWaves : 1;
    u32x4 k_r[KI];
    if constexpr (KLDS) {
#pragma unroll
        for (int kk = 0; kk < KI; ++kk) {
            const int u = min(wave + kk * kLargeWaves, NP / 4 - 1);
            const int row = 4 * u + (lane >> 4), pc = lane & 15;
            const int srow = min(row, max(n - 1, 0));
            k_r[kk] = *reinterpret_cast<const u32x4*>(Kb + (size_t)srow * kq_row + ((pc ^ (row & 15)) << 3));
        }
    }
    // (the tree's values are used only below: their arithmetic may not be
    // moved up to the loads, where it would wait for them before the other
    // requests are out)
#pragma unroll
    for (int k = 0; k < PL; ++k) asm volatile("" : "+v"(par_r[k]), "+v"(g_r[k]), "+v"(beta_r[k]));
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
                const int i = x >> 4, c = cbase + 16 * wave + (x & 15);
                if (i < n) O[vo_base + (size_t)i * vo_row + c] = 0x7fc0;
                Ug[(size_t)i * kD + c] = qnan;
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
    int32_t* s_fc = reinterpret_cast<int32_t*>(s_cm + (NP + 1) * WC);   // [NP + 1] first child, -1: none
    int32_t* s_nx = s_fc + (NP + 1);                    // [NP] node after the subtree (n: none; -1 pending)
    int32_t* s_ptr = s_nx + NP;                         // [NP] doubling link
    int32_t* s_rk = s_ptr + NP;                         // [NP] list distance to the last node
    int32_t* s_sc = s_rk + NP;                          // [NP] list link (n: past the last node)
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
    if constexpr (KLDS) {
#pragma unroll
        for (int kk = 0; kk < KI; ++kk) {
            const int u = wave + kk * kLargeWaves;
            if (u < NP / 4) *reinterpret_cast<u32x4*>(s_k + 4 * u * kD + 8 * lane) = k_r[kk];
        }
    }
    // the slice's S0 rows as bf16 (row c at LDS row c, chunks swizzled)
#pragma unroll
    for (int k = 0; k < S0L; ++k) {
        const int x = tid + k * NT;
        if (x < 64 * kD / 4) {
            const int r = x >> 5, c4 = x & 31;          // row, float4 within the row
            uint2 w;
            w.x = (uint32_t)bf16_rne(s0_r[k].x) | ((uint32_t)bf16_rne(s0_r[k].y) << 16);
            w.y = (uint32_t)bf16_rne(s0_r[k].z) | ((uint32_t)bf16_rne(s0_r[k].w) << 16);
            *reinterpret_cast<uint2*>(s_s0 + row_chunk(r, c4 >> 1) + 4 * (c4 & 1)) = w;
        }
    }
    if (tid < 9) s_more[tid] = 0;
    if (tid < NB) s_xready[tid] = 0;
    if (tid < kSolveWaves) s_uready[tid] = 0;
    // a chain skips the construction (nt = 0): the identity and last = n - 1
    if (not_chain) s_notchain = 1;
    lds_barrier();
    const int nt = s_notchain ? n : 0;
    for (int i = tid; i < nt; i += NT) {                // bit i of its parent's children row
        const int p = s_jump[i];
        atomicOr(&s_cm[(p < 0 ? NP : p) * WC + (i >> 5)], 1u << (i & 31));
    }
    lds_barrier();
    for (int v = tid; v <= NP; v += NT) {               // first child (row NP: the first root)
        int f = -1;
        if (v < nt || v == NP)
            for (int w = 0; w < WC; ++w) {
                const uint32_t x = s_cm[v * WC + w];
                if (x) {
                    f = 32 * w + __builtin_ctz(x);
                    break;
                }
            }
        s_fc[v] = f;
    }
    for (int i = tid; i < nt; i += NT) {                // next sibling, else pending
        const int p = s_jump[i];
        const uint32_t* r = s_cm + (p < 0 ? NP : p) * WC;
        int nsib = -1;
        uint32_t x = r[i >> 5] & ~((2u << (i & 31)) - 1u);   // siblings above i in its word
        for (int w = i >> 5;;) {
            if (x) {
                nsib = 32 * w + __builtin_ctz(x);
                break;
            }
            if (++w >= WC) break;
            x = r[w];
        }
        s_nx[i] = nsib >= 0 ? nsib : (p < 0 ? n : -1);
        s_ptr[i] = p;
    }
    lds_barrier();
    // the node after a subtree: the subtree root's next sibling, else its
    // parent's (pointer doubling up the path; a root-level node always has one)
    for (int rd = 0;; ++rd) {
        int res[PL], nq[PL];
        bool more = false;
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            res[k] = -2;
            nq[k] = 0;
            if (i < nt && s_nx[i] < 0) {
                const int q = s_ptr[i];
                const int rq = s_nx[q];
                if (rq >= 0) res[k] = rq;
                else {
                    nq[k] = s_ptr[q];
                    res[k] = -1;
                    more = true;
                }
            }
        }
        if (tid == 0) s_more[(rd + 1) % 3] = 0;
        lds_barrier();
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            if (res[k] >= 0) s_nx[i] = res[k];
            else if (res[k] == -1) s_ptr[i] = nq[k];
        }
        if (more) s_more[rd % 3] = 1;
        lds_barrier();
        if (!s_more[rd % 3]) break;
    }
    for (int i = tid; i < nt; i += NT) {                // preorder successor: first child, else the node after
        const int f = s_fc[i];
        const int sc = f >= 0 ? f : s_nx[i];
        s_sc[i] = sc;
        s_rk[i] = sc < n ? 1 : 0;
    }
    lds_barrier();
    for (int rd = 0;; ++rd) {                           // list ranking by pointer doubling
        int nr[PL], ns[PL];
        bool more = false;
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            nr[k] = -1;
            ns[k] = n;
            if (i < nt) {
                const int sc = s_sc[i];
                if (sc < n) {
                    nr[k] = s_rk[i] + s_rk[sc];
                    ns[k] = s_sc[sc];
                    more |= ns[k] < n;
                }
            }
        }
        if (tid == 0) s_more[3 + (rd + 1) % 3] = 0;
        lds_barrier();
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            if (nr[k] >= 0) {
                s_rk[i] = nr[k];
                s_sc[i] = ns[k];
            }
        }
        if (more) s_more[3 + rd % 3] = 1;
        lds_barrier();
        if (!s_more[3 + rd % 3]) break;
    }
    for (int i = tid; i < nt; i += NT) {                // position n - 1 - rank
        const int pi = min(max(n - 1 - s_rk[i], 0), n - 1);
        const int nx = s_nx[i];
        s_perm[pi] = (uint16_t)i;
        s_last[pi] = (int16_t)((nx < n ? n - 1 - s_rk[nx] : n) - 1);
    }
    lds_barrier();
    // ancestor rows from the preorder: j is a strict ancestor of r exactly when
    // pos(j) < pos(r) <= last(pos(j)), and only j < r can be one.  Each node's
    // (pos, last) is packed once into the free children-row scratch (nodes
    // past the tree get pos 0xffff, never below a row's position); the tree's
    // workgroups share the (row, word) pairs, one pair per thread.
    const int nparts = Hv * 2, part = h * 2 + slice;
    {
        uint32_t* pk = s_cm;
        for (int j = tid; j < NP; j += NT) {
            uint32_t v = 0xffffu;
            if (j < n) {
                const int pj = nt ? min(max(n - 1 - s_rk[j], 0), n - 1) : j;
                v = (uint32_t)pj | ((uint32_t)(uint16_t)s_last[pj] << 16);
            }
            pk[j] = v;
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
    }
    auto node_at = [&](int pos) __attribute__((always_inline)) {   // position (clamped) -> node
        return min((int)s_perm[min(pos, n - 1)], n - 1);
    };
    for (int sb = tid; sb < NB; sb += NT) {
        int m = -1;
        for (int e = 0; e < 16; ++e) m = max(m, (int)s_last[16 * sb + e]);
        s_mlast[sb] = m;
    }

    // path log-gates.  A chain's are prefix sums: a scan within each wave
    // (lane shifts) and the preceding waves' totals.  Any other tree's by
    // synchronous pointer doubling (each node adds its link's sum and jumps
    // to the link's link); round r raises flag r % 3 while a node still has a
    // link to follow and clears flag (r + 1) % 3 before its first barrier: two
    // LDS-only barriers per round
    if (nt == 0) {
        static_assert(NP <= NT, "one chain node per thread");
        float x = tid < NP ? s_lg[tid] : 0.f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        // (past the preorder's scratch, whose packed rows may still be read)
        float* wsum = reinterpret_cast<float*>(reinterpret_cast<char*>(s_big) + SCRATCH);
        static_assert(SCRATCH + 4 * kLargeWaves <= BIG, "wave sums fit the ring area");
        if (lane == 63) wsum[wave] = x;
        lds_barrier();
        for (int w = 0; w < wave; ++w) x += wsum[w];
        if (tid < NP) {
            s_lg[tid] = x;
            s_hop[tid] = (int16_t)(tid < n ? tid + 1 : 0);
        }
        lds_barrier();
    }
    for (int rd = 0; nt; ++rd) {
        int nn[PL], hj[PL];
        float gj[PL];
        bool more = false;
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            const int j = i < NP ? s_jump[i] : -1;
            nn[k] = j >= 0 ? s_jump[j] : -1;
            gj[k] = j >= 0 ? s_lg[j] : 0.f;
            hj[k] = j >= 0 ? s_hop[j] : 0;
            more |= nn[k] >= 0;
        }
        if (tid == 0) s_more[6 + (rd + 1) % 3] = 0;
        lds_barrier();
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int i = tid + k * NT;
            if (i < NP && s_jump[i] >= 0) {
                s_lg[i] += gj[k];
                s_hop[i] = (int16_t)(s_hop[i] + hj[k]);
                s_jump[i] = nn[k];
            }
        }
        if (more) s_more[6 + rd % 3] = 1;
        lds_barrier();
        if (!s_more[6 + rd % 3]) break;
    }
    if (slice == 0)
        for (int i = tid; i < n; i += NT) a.log_gamma[((size_t)b * Hv + h) * N + i] = s_lg[i];
    for (int r = part + nparts * tid; r < N; r += nparts * NT)   // depth: the rows' shares again
        a.depth[(size_t)b * N + r] = r < n ? s_hop[r] - 1 : -1;

    // G and beta by position (through the scratch: the ring area is free; a
    // chain is in position order already)
    if (nt) {
        float* tl = reinterpret_cast<float*>(s_big);
        float* tb = tl + NP;
        for (int i = tid; i < NP; i += NT) {
            const int v = node_at(i);
            tl[i] = i < n ? s_lg[v] : 0.f;
            tb[i] = i < n ? s_beta[v] : 0.f;
        }
        lds_barrier();
        for (int i = tid; i < NP; i += NT) {
            s_lg[i] = tl[i];
            s_beta[i] = tb[i];
        }
    }
    // occupancy: tile (t, s), s < t, holds an ancestor pair exactly when a
    // position of block s has its subtree reaching row t.  Row t's tiles in
    // ascending s, so the tile of the block just before it (the one that
    // waits for the previous row's U) comes last.
    for (int t = tid; t < NB; t += NT) {
        int m = 0;
        for (int sb = 0; sb < t && t < nblk; ++sb)
            if (s_mlast[sb] >= 16 * t) s_tcol[t][m++] = (uint8_t)sb;
        s_tn[t] = m;
    }
    lds_barrier();
    // the ring: row t takes the next 8 + s_tn[t] slots, rounded up to an even
    // count so that 2-slot objects never wrap (counted over all rows, modulo
    // RING); they may be written once every row whose slots they reuse has
    // been consumed by all solve waves.  One wave, row r in lane r.
    lds_barrier();
    if (wave == 0) {
        const int tn = lane < nblk ? s_tn[lane] : 0;
        const int sl = lane < nblk ? 8 + tn + (tn & 1) : 0;
        int inc = sl;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(inc, d);
            if (lane >= d) inc += y;
        }
        const int gsl = inc - sl;                       // first slot of row lane; lane nblk: the total
        const int target = inc - RING;                  // rows starting below it must be consumed
        int cnt = 0;
        for (int r = 0; r < nblk; ++r) {
            const int gr = __builtin_amdgcn_readlane(gsl, r);
            cnt += (r < lane && gr < target) ? 1 : 0;
        }
        if (lane <= NB) s_gslot[lane] = gsl;
        if (lane < NB) s_rstar[lane] = cnt;
    }
    lds_barrier();
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};

    // k / q fragment of node block blk, column chunk cs: lane (r, q) holds
    // row 16 blk + r (clamped), columns 32 cs + 8 q .. +7.  From global
    // memory (a uniform base and a 32-bit lane offset) or, for k, from LDS.
    const uint32_t lane_col = 16u * lq;
    auto gfrag = [&](const uint16_t* base, int blk, int cs) __attribute__((always_inline)) {
        const uint32_t row = (uint32_t)node_at(16 * blk + ln);
        const uint32_t off = row * (uint32_t)(kq_row * 2) + lane_col + 64u * cs;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              reinterpret_cast<const char*>(base) + off));
    };
    auto kfrag = [&](int blk, int cs) __attribute__((always_inline)) {
        if constexpr (KLDS) {
            const int row = node_at(16 * blk + ln);
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s_k + row_chunk(row, 4 * cs + lq)));
        } else {
            return gfrag(Kb, blk, cs);
        }
    };
    // S0 rows col0 + r of the slice: lane (r, q) holds columns 32 cs + 8 q ..
    // +7; the same registers are the B operand S0^T (for K S0^T) and the A
    // operand S0 (for S0 Q^T)
    auto s0frag = [&](int col0, int cs) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(s_s0 + row_chunk(col0 + ln, 4 * cs + lq)));
    };
    // ring slot x, as 8-byte (tiles) or 16-byte (right-hand sides) lane words
    uint2* ring8 = s_big;
    u32x4* ring16 = reinterpret_cast<u32x4*>(s_big);
    auto slot_at = [&](int x) __attribute__((always_inline)) { return x < RING ? x : x - RING; };

    // Nothing of the setup is in flight past this point (its loads are
    // consumed; its cache stores have long completed), so the loops below
    // start from an empty count and the compiler's waits in them count only
    // their own requests.
    wait_vmem_all();
    if (solver) {
        // ================= solve waves =================
        const int g = wave;
        const int c0 = cbase + 16 * g;                  // this wave's first value column
        const __amdgpu_buffer_rsrc_t u_rsrc =
            __builtin_amdgcn_make_buffer_rsrc(Ug, (short)0, N * kD * 4, kBufferFlags);
        s16x4 uprev = {0, 0, 0, 0};
        for (int t = 0; t < nblk; ++t) {
            const int nts = s_tn[t];
            const int base = s_gslot[t] % RING;
            wait_flag_ge(&s_xready[t], 1);
            // D_t R_t of this group: 16 bytes per lane in slot base + 2g
            f32x4 acc = __builtin_bit_cast(f32x4, ring16[slot_at(base + 2 * g) * 32 + lane]);
            // U_t = D_t R_t - sum_s X~_ts U_s (the tiles hold -X~); four tiles'
            // operands are read before their products
            int sl = slot_at(base + 8);
            f32x4 acc2 = z;
            int m = 0;
            for (; m + 4 <= nts; m += 4) {
                s16x4 xa[4], ub[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = __builtin_amdgcn_readfirstlane((int)s_tcol[t][m + e]);
                    xa[e] = __builtin_bit_cast(s16x4, ring8[slot_at(sl + e) * 64 + lane]);
                    ub[e] = s == t - 1 ? uprev : __builtin_bit_cast(s16x4, s_u[s][g][lane]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (e & 1) acc2 = mfma16(xa[e], ub[e], acc2);
                    else acc = mfma16(xa[e], ub[e], acc);
                }
                sl = slot_at(sl + 4);
            }
            for (; m < nts; ++m) {
                const int s = __builtin_amdgcn_readfirstlane((int)s_tcol[t][m]);
                const s16x4 xa = __builtin_bit_cast(s16x4, ring8[sl * 64 + lane]);
                const s16x4 ub = s == t - 1 ? uprev : __builtin_bit_cast(s16x4, s_u[s][g][lane]);
                acc = mfma16(xa, ub, acc);
                sl = slot_at(sl + 1);
            }
            acc += acc2;
            uprev = to_bf16x4(acc);
            s_u[t][g][lane] = __builtin_bit_cast(uint2, uprev);
            publish_set(&s_uready[g], t + 1, lane);    // also frees row t's ring slots
            // the cache row: lane (n, q) holds rows 4q .. 4q+3 of column n;
            // positions past the tree store outside the buffer and are dropped
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                const int i = 16 * t + 4 * lq + mm;
                const int off = i < n ? (node_at(i) * kD + c0 + ln) * 4 : 0x7fffffff;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[mm]), u_rsrc, off, 0, 0);
            }
        }
        return;
    }

    // ================= row owners =================
    const int p = wave - kSolveWaves;                   // 0 .. kOwners - 1
    // o rows of this tree and head: node v's row at v Hv kD elements
    const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        O + vo_base, (short)0, ((n - 1) * Hv + 1) * kD * 2, kBufferFlags);
    const uint16_t* Vb = static_cast<const uint16_t*>(a.v) + vo_base + cbase;   // (+ 4 lq per lane below)
    s16x4 ident;
#pragma unroll
    for (int e = 0; e < 4; ++e) ident[e] = (4 * lq + e == ln) ? (short)0x3f80 : (short)0;
    for (int t = p; t < nblk; t += kOwners) {
        const int nts = s_tn[t];
        // operands, requested before the wait for ring space: k of the row,
        // its v rows for the four groups (lane (r, q): columns 16 gg + 4q ..
        // +3 of row r) and, when k comes from global memory, k of its first
        // kChunk occupied blocks (from LDS they are read tile by tile)
        bf16x8 kt[4], kx[kChunk][4];
        uint2 vt[4];
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) kt[cs] = kfrag(t, cs);
        {
            const uint32_t vr = (uint32_t)node_at(16 * t + ln) * (uint32_t)(vo_row * 2);   // (bytes, a uniform base)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg)
                vt[gg] = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(Vb) + vr + 8u * lq + 32u * gg);
        }
        // k of the occupied blocks m0 .. m0 + kChunk - 1 (past the row's: its own)
        auto load_chunk = [&](int m0) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                const int s = m0 + e < nts ? (int)s_tcol[t][m0 + e] : t;
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) kx[e][cs] = kfrag(s, cs);
            }
        };
        if constexpr (!KLDS) load_chunk(0);             // (from LDS: after the inverse, fewer live registers)
        // this row's nodes (rows 4q .. 4q+3 of the accumulator layout)
        float bei[4], lgi4[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            bei[m] = s_beta[16 * t + 4 * lq + m];
            lgi4[m] = s_lg[16 * t + 4 * lq + m];
        }
#pragma unroll
        for (int gg = 0; gg < kSolveWaves; ++gg) wait_flag_ge(&s_uready[gg], s_rstar[t]);
        const int base = s_gslot[t] % RING;
        // ---- D_t = (I + X_tt)^-1, with the row's right-hand-side slots as
        // scratch (X_tt in fp32 at slot base, D as an A operand at base + 2) ----
        float* xd = reinterpret_cast<float*>(&ring8[base * 64]);
        uint16_t* dd = reinterpret_cast<uint16_t*>(&ring8[slot_at(base + 2) * 64]);
        {
            f32x4 gr = z;
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) gr = mfma32(kt[cs], kt[cs], gr);   // lane (j, q): [i = 4q + m][j]
            const int pj = 16 * t + ln;
            const int lj = s_last[pj];
            const float lgj = s_lg[pj];
            float4 xv;
            float* xp = reinterpret_cast<float*>(&xv);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int pi = 16 * t + 4 * lq + m;
                const bool anc = (pj < pi) & (pi <= lj);
                const float x = bei[m] * __expf(fminf(lgi4[m] - lgj, 0.f)) * gr[m];
                xp[m] = anc ? x : 0.f;
            }
            *reinterpret_cast<float4*>(&xd[ln * 16 + 4 * lq]) = xv;      // [col j][row i]
            // fp32 forward substitution, four lanes per column: lane 4c + qd
            // holds rows 4qd .. 4qd+3 of column c; step m broadcasts y_m from
            // its owner within the lane quad and updates the rows below it
            const int c = lane >> 2, qd = lane & 3;
            float accd[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) accd[e] = (4 * qd + e == c) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                const float4 xc = *reinterpret_cast<const float4*>(&xd[m * 16 + 4 * qd]);
                const float ym = quad_bcast(accd[m & 3], m >> 2);
                const float xr[4] = {xc.x, xc.y, xc.z, xc.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {                 // rows below m only
                    const float upd = fmaf(-xr[e], ym, accd[e]);
                    accd[e] = 4 * qd + e > m ? upd : accd[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) dd[a16_pos(4 * qd + e, c)] = bf16_rne(accd[e]);
        }
        const s16x4 dt = __builtin_bit_cast(s16x4, reinterpret_cast<const uint2*>(dd)[lane]);   // A: D; B: D^T
        // ---- the row's -X~ tiles, kChunk at a time (their reads and products
        // independent of each other) ----
        for (int m0 = 0; m0 < nts; m0 += kChunk) {
            if (m0 > 0 || KLDS) load_chunk(m0);
            int sc[kChunk];
            f32x4 gr[kChunk];
            int lj[kChunk];
            float lgj[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                sc[e] = m0 + e < nts ? __builtin_amdgcn_readfirstlane((int)s_tcol[t][m0 + e]) : t;
                lj[e] = s_last[16 * sc[e] + ln];
                lgj[e] = s_lg[16 * sc[e] + ln];
                gr[e] = z;
            }
#pragma unroll
            for (int cs = 0; cs < 4; ++cs)
#pragma unroll
                for (int e = 0; e < kChunk; ++e) gr[e] = mfma32(kt[cs], kx[e][cs], gr[e]);   // lane (j, q): [i = 4q + m][j]
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                s16x4 xa;                               // X^T as an A operand
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const int pi = 16 * t + 4 * lq + mm;
                    const bool anc = (sc[e] < t) & (pi <= lj[e]);   // (pj < pi: s < t)
                    const float x = bei[mm] * __expf(fminf(lgi4[mm] - lgj[e], 0.f)) * gr[e][mm];
                    xa[mm] = (short)bf16_rne(anc ? x : 0.f);
                }
                const f32x4 xt = mfma16(xa, dt, z);     // X^T D^T: lane (i, q) holds X~[i][4q + m]
                s16x4 nx;
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) nx[mm] = (short)bf16_rne(-xt[mm]);
                if (m0 + e < nts) ring8[slot_at(base + 8 + m0 + e) * 64 + lane] = __builtin_bit_cast(uint2, nx);
            }
        }
        bf16x8 qt[4];                                   // q of the row, for the outputs
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) qt[cs] = gfrag(Qb, t, cs);
        // ---- D_t R_t of the four groups, R_t = diag(beta)(V_t - diag(e^G) K_t S0^T);
        // V moves into the accumulator layout by an exact product with I ----
        f32x4 rt[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            f32x4 ks = z;
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) ks = mfma32(kt[cs], s0frag(16 * gg, cs), ks);   // [node][col]
            const f32x4 vd = mfma16(__builtin_bit_cast(s16x4, vt[gg]), ident, z);
            f32x4 R;
#pragma unroll
            for (int m = 0; m < 4; ++m) R[m] = bei[m] * (vd[m] - __expf(lgi4[m]) * ks[m]);
            s16x4 rh, rl;
            split4(R, rh, rl);
            rt[gg] = mfma16(dt, rl, mfma16(dt, rh, z));
        }
        // (the scratch in slots base .. base + 2 is read: D is in registers)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) ring16[slot_at(base + 2 * gg) * 32 + lane] = __builtin_bit_cast(u32x4, rt[gg]);
        publish_set(&s_xready[t], 1, lane);
        // (q is used only below this point: its products may not be moved
        // ahead of the publication, which would then wait for its loads)
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) asm volatile("" : "+v"(qt[cs]));
        // ---- outputs O_t = e^G Q_t S0^T + sum_{s <= t} Y_ts U_s ----
        f32x4 oc[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            oc[gg] = z;
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) oc[gg] = mfma32(s0frag(16 * gg, cs), qt[cs], oc[gg]);   // [col][node]
        }
        const int pi = 16 * t + ln;                     // this lane's node (column of the products)
        const float lgi = s_lg[pi];
        const float egi = __expf(lgi);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) oc[gg] *= egi;
        // Y tiles four at a time: their Gram products first, then the wait for
        // the last of their rows of U (rows are published in order), then the
        // products with U of every column group
        auto y_group = [&](const int (&sc)[kChunk], int cnt, const bf16x8 (&ks)[kChunk][4]) __attribute__((always_inline)) {
            f32x4 gr[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) gr[e] = z;
#pragma unroll
            for (int cs = 0; cs < 4; ++cs)
#pragma unroll
                for (int e = 0; e < kChunk; ++e) gr[e] = mfma32(ks[e][cs], qt[cs], gr[e]);   // lane (i, q): [j = 4q + m][i]
            s16x4 yb[kChunk];                           // Y^T as B operands
#pragma unroll
            for (int e = 0; e < kChunk; ++e)
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const int pj = 16 * sc[e] + 4 * lq + mm;
                    const int lpj = s_last[pj];
                    const bool anc = (e < cnt) & (pj <= pi) & (pi <= lpj);
                    const float y = __expf(fminf(lgi - s_lg[pj], 0.f)) * gr[e][mm];
                    yb[e][mm] = (short)bf16_rne(anc ? y : 0.f);
                }
            int smax = sc[0];
#pragma unroll
            for (int e = 1; e < kChunk; ++e) smax = e < cnt ? max(smax, sc[e]) : smax;
#pragma unroll
            for (int gg = 0; gg < kSolveWaves; ++gg) wait_flag_ge(&s_uready[gg], smax + 1);
#pragma unroll
            for (int e = 0; e < kChunk; ++e)
                if (e < cnt)
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg)
                        oc[gg] = mfma16(__builtin_bit_cast(s16x4, s_u[sc[e]][gg][lane]), yb[e], oc[gg]);
        };
        // the occupied blocks s < t, then the diagonal block (its wait is for
        // the solve's row t)
        const int nall = nts + 1;
        for (int m0 = 0; m0 < nall; m0 += kChunk) {
            // (a single chunk of tiles is still in registers, and past the row's
            // blocks it holds the row's own; a diagonal block left alone in a
            // chunk of its own takes the row's k)
            if (nts > kChunk || (KLDS && nts == 0)) {
                load_chunk(m0);
            } else if (m0 > 0) {
#pragma unroll
                for (int e = 0; e < kChunk; ++e)
#pragma unroll
                    for (int cs = 0; cs < 4; ++cs) kx[e][cs] = kt[cs];
            }
            int sc[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                const int m = m0 + e;
                sc[e] = m < nts ? __builtin_amdgcn_readfirstlane((int)s_tcol[t][m]) : t;
            }
            y_group(sc, min(kChunk, nall - m0), kx);
        }
        // (positions past the tree store outside the buffer and are dropped)
        const int orow = pi < n ? (node_at(pi) * Hv * kD + cbase + 4 * lq) * 2 : 0x7fffffff;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            u32x2 w;
            w[0] = (uint32_t)bf16_rne(oc[gg][0]) | ((uint32_t)bf16_rne(oc[gg][1]) << 16);
            w[1] = (uint32_t)bf16_rne(oc[gg][2]) | ((uint32_t)bf16_rne(oc[gg][3]) << 16);
            __builtin_amdgcn_raw_buffer_store_b64(w, o_rsrc, orow + 32 * gg, 0, 0);
        }
    }
}

}  // namespace

bool verify_large_supported(const VerifyArgs& a, int io) {
    return io == GDN_BF16 && a.dk == kD && a.dv == kD && a.N > 128 && a.N <= kLargeMaxN;
}

hipError_t launch_verify_large(const VerifyArgs& a, int io, hipStream_t stream) {
    (void)io;
    VerifyArgs copy = a;
    // two 64-column slices per (sequence, value head); a unit's slices are
    // 8 workgroups apart, so both run on one XCD
    int units = a.B * a.Hv;
    const unsigned grid = 16u * (unsigned)((units + 7) / 8);
    const void* fn = a.N <= 256 ? (const void*)verify_large_kernel<16> : (const void*)verify_large_kernel<32>;
    void* args[] = {&copy, &units};
    return hipLaunchKernel(fn, dim3(grid), dim3(kLargeThreads), args, 0, stream);
}

}  // namespace gdn
