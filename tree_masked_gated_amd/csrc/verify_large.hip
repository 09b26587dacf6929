// verify_large.hip -- MFMA tree verification for d_k = d_v = 128, bf16
// q/k/v/o and trees of 129 .. 16 * NB nodes (NB = 16 or 32 blocks of 16 nodes).
//
// Same method as the small-tree kernel (page "Trees from Marginals:
// Autoregressive drafting with factorized priors", section 3: the Gram matrix,
// a tiled forward substitution and the output stage, fused), laid out for trees
// whose k / q rows and interaction tiles no longer fit in LDS together, in
// one launch: verify_large_kernel, one workgroup per (sequence, value head,
// column slice), checks the parent row and relabels the tree's nodes in
// preorder (every subtree one run of positions, so ancestry is an interval
// test and a block row's ancestors sit in few column blocks; one workgroup
// per tree writes the ancestor rows, depth and status from it).  It walks the
// 16-position block rows t in order: for each row it computes only the Gram
// tiles (t, s) that hold an ancestor pair, spread over the waves, into an LDS
// row buffer (two of them, alternating), and the solve waves run the row's
// blocked substitution and output stage for their value columns, two blocks
// per MFMA.  Row t + 1's tiles are computed while row t is solved, so one
// barrier per row separates them.  Inputs are gathered and outputs written at
// the caller's node indices.
// k / q rows are read from global memory (L2) straight into MFMA operand
// registers, a row ahead of their use.
#include "gdn_common.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"

namespace gdn {

namespace {

constexpr int kLargeMaxN = 512;      // largest tree of this path

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

// Waves 0 .. NS-1 solve: wave w owns value columns 64 slice + 16 CG w .. as CG
// 16-column groups (with two, two independent MFMA chains per product).  Waves
// NS .. NS+NG-1 are Gram waves: they compute the next block row's tiles and (the
// last NCG of them, one 16-column group each) its projections K_t S0^T and
// S0 Q_t^T into LDS, while the solve waves run the current row; one barrier
// per row.  The two roles run separate loops with the same barrier count, so
// neither keeps the other's registers.
template <int NB>
__global__ __launch_bounds__(512, 1) void verify_large_kernel(VerifyArgs a, int csplit) {
    constexpr int NP = 16 * NB;                 // padded node count
    constexpr int NT = 512;
    // solve waves hold their U blocks in registers (CG * NB / 2 stacked
    // pairs): 512-node trees split the columns over four solve waves so each
    // keeps room for loads in flight, leaving four Gram waves (a preorder row
    // has few tiles)
    constexpr int NS = NB > 16 ? 4 : 2;         // solve waves, 16 CG value columns each
    constexpr int NG = 8 - NS;                  // Gram waves
    constexpr int NCG = 4;                      // 16-column groups per workgroup
    constexpr int CG = NCG / NS;                // groups per solve wave
    static_assert(NS * CG == NCG && NG >= NCG, "column groups cover the slice; every group has a projection wave");
    constexpr int NPR = NB / 2;                 // U pairs
    constexpr int TPW = 3;                      // tiles per Gram wave requested a row ahead
    constexpr int KC = 16;                      // node blocks whose k rows are cached in LDS
    constexpr bool KALL = NB <= KC;             // every block cached: no k rows from L2 in the Gram
    // -X and Y tiles of one block row, by column block s, for rows of either
    // parity; a spare tile at the end (a pair read may run 512 bytes past the
    // last tile; those lanes are zeroed before use)
    __shared__ __attribute__((aligned(16))) uint16_t s_xrow[2][NB * 256 + 256];
    __shared__ __attribute__((aligned(16))) uint16_t s_yrow[2][NB * 256 + 256];
    __shared__ __attribute__((aligned(16))) uint16_t s_dinv[2][256];
    __shared__ __attribute__((aligned(16))) float s_xd[2][256];
    __shared__ __attribute__((aligned(16))) f32x4 s_pk[2][NCG][64];   // K_t S0^T, accumulator layout
    __shared__ __attribute__((aligned(16))) f32x4 s_pq[2][NCG][64];   // S0 Q_t^T
    __shared__ __attribute__((aligned(16))) float s_lg[NP];
    __shared__ __attribute__((aligned(16))) float s_beta[NP];
    __shared__ __attribute__((aligned(16))) int32_t s_jump[NP];
    __shared__ unsigned long long s_occ[NB];    // bit s of row t: tile (t, s), s < t, not all zero
    __shared__ uint8_t s_tcol[NB][NB];          // row t's tiles: t, then its occupied blocks s < t, descending
    __shared__ int s_more[9];                   // per-round flags of the three doubling loops (3 each)
    // the node order the kernel works in: a preorder (every subtree one run of
    // positions), position -> node, and each position's last descendant
    __shared__ uint16_t s_perm[NP];
    __shared__ __attribute__((aligned(8))) int16_t s_last[NP];
    __shared__ int s_mlast[NB];                 // largest s_last of each 16-position block
    __shared__ int s_bad;                       // first node with an invalid parent
    __shared__ int16_t s_hop[NP];               // nodes on the path to the root (depth + 1), by doubling
    // k rows of blocks 0 .. KC-1 in MFMA operand order: (block s, chunk cs) is
    // 1 KB, lane l's 16 bytes at l * 16 (row 16 s + l % 16, columns 32 cs +
    // 8 (l / 16) .. +7), so a fragment read is one conflict-free ds_read_b128
    __shared__ __attribute__((aligned(16))) uint16_t s_kc[KC * 4 * 512];

    const int N = a.N, Hv = a.Hv, Hk = a.Hk, G = Hv / Hk;
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool solver = wave < NS;
    const int item = blockIdx.x;
    const int slice = item % csplit, bh = item / csplit;
    const int h = bh % Hv, b = bh / Hv, hk = h / G;
    const int cbase = slice * (16 * NCG);               // the workgroup's first value column
    // this tree's rows in the node arrays (n nodes); the cache keeps N rows per tree
    const SeqRows rows = seq_rows(a.offsets, b, N);
    const int n = max(rows.n, 0);
    const int nblk = (n + 15) / 16;
    const size_t vo_row = (size_t)Hv * kD;
    const size_t vo_base = (rows.row0 * Hv + h) * kD;
    uint16_t* O = static_cast<uint16_t*>(a.o);
    float* Ug = a.u + ((size_t)b * Hv + h) * (size_t)N * kD;

    // tree check, the same in every workgroup of the tree: 0, or one plus the
    // first node whose parent is outside [-1, i); -1 for rows past the
    // batch's offsets.  For an invalid or empty tree one workgroup publishes
    // zero ancestor rows, depth -1 and the status; a valid tree's rows and
    // depths are shared out once its preorder is known.
    const int W = (N + 31) / 32;
    const bool writer = h == 0 && slice == 0;
    uint32_t* gm = a.anc_mask + (size_t)b * N * W;
    if (tid == 0) s_bad = 0x7fffffff;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
        const int p = a.parent[rows.row0 + i];
        if (p < -1 || p >= i) atomicMin(&s_bad, i);
    }
    __syncthreads();
    const int status = rows.n < 0 ? -1 : s_bad == 0x7fffffff ? 0 : s_bad + 1;
    if (writer && (status || n == 0)) {
        for (int x = tid; x < N * W; x += NT) gm[x] = 0u;
        for (int r = tid; r < N; r += NT) a.depth[(size_t)b * N + r] = -1;
        if (tid == 0) a.status[b] = status;
    }
    if (status) {                                       // invalid tree: NaN outputs
        const float qnan = __uint_as_float(0x7fc00000u);
        if (solver)
            for (int x = lane; x < N * 16 * CG; x += 64) {
                const int i = x / (16 * CG), c = cbase + 16 * CG * wave + x % (16 * CG);
                if (i < n) O[vo_base + (size_t)i * vo_row + c] = 0x7fc0;
                Ug[(size_t)i * kD + c] = qnan;
            }
        if (slice == 0)
            for (int i = tid; i < N; i += NT) a.log_gamma[((size_t)b * Hv + h) * N + i] = qnan;
        return;
    }
    if (n == 0) return;                                 // an empty tree: nothing to verify

    const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + (rows.row0 * Hk + hk) * kD;
    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + (rows.row0 * Hk + hk) * kD;
    const size_t kq_row = (size_t)Hk * kD;
    // ---- a preorder of the tree, path log-gates G, beta, tile occupancy ----
    // In a preorder (children in index order) j is a strict ancestor of i
    // exactly when j < i <= last(j), last(j) the position of j's last
    // descendant, so a block row's ancestors sit in few column blocks (a
    // random tree's rows touch most blocks in the caller's order) and the
    // tile masks need no ancestor rows.  Outputs stay in the caller's order.
    // Scratch while it is built: the X / Y row buffers.
    constexpr int WC = NP / 32;                         // words of a children row
    constexpr int PER = NP / NT > 0 ? NP / NT : 1;
    uint32_t* s_cm = reinterpret_cast<uint32_t*>(&s_xrow[0][0]);  // [NP + 1][WC]; row NP: the roots
    int32_t* s_fc = reinterpret_cast<int32_t*>(&s_yrow[0][0]);    // [NP + 1] first child, -1: none
    int32_t* s_nx = s_fc + (NP + 1);                    // [NP] node after the subtree (n: none; -1 pending)
    int32_t* s_ptr = s_nx + NP;                         // [NP] doubling link
    int32_t* s_rk = s_ptr + NP;                         // [NP] list distance to the last node
    int32_t* s_sc = s_rk + NP;                          // [NP] list link (n: past the last node)
    static_assert((NP + 1) * WC * 4 <= sizeof(s_xrow) && (5 * NP + 1) * 4 <= sizeof(s_yrow),
                  "preorder scratch fits the row buffers");
    bool not_chain = false;                             // a chain is its own preorder
    for (int i = tid; i < NP; i += NT) {
        const bool v = i < n;
        const int p = v ? a.parent[rows.row0 + i] : -1;
        not_chain |= v && p != i - 1;
        s_jump[i] = p;
        s_lg[i] = v ? logf(a.g[(rows.row0 + i) * Hv + h]) : 0.f;
        s_beta[i] = v ? a.beta[(rows.row0 + i) * Hv + h] : 0.f;
        s_perm[i] = (uint16_t)min(i, max(n - 1, 0));
        s_last[i] = v ? (int16_t)(n - 1) : (int16_t)-1;
        s_hop[i] = v ? (int16_t)1 : (int16_t)0;
    }
    for (int x = tid; x < (NP + 1) * WC; x += NT) s_cm[x] = 0u;
    if (tid < 9) s_more[tid] = 0;
    // a chain skips the construction (nt = 0): the identity and last = n - 1
    const int nt = __syncthreads_or(not_chain) ? n : 0;
    for (int i = tid; i < nt; i += NT) {                // bit i of its parent's children row
        const int p = s_jump[i];
        atomicOr(&s_cm[(p < 0 ? NP : p) * WC + (i >> 5)], 1u << (i & 31));
    }
    __syncthreads();
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
    __syncthreads();
    // the node after a subtree: the subtree root's next sibling, else its
    // parent's (pointer doubling up the path; a root-level node always has one)
    for (int rd = 0;; ++rd) {
        int res[PER], nq[PER];
        bool more = false;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
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
        for (int k = 0; k < PER; ++k) {
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
    __syncthreads();
    for (int rd = 0;; ++rd) {                           // list ranking by pointer doubling
        int nr[PER], ns[PER];
        bool more = false;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
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
        for (int k = 0; k < PER; ++k) {
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
    __syncthreads();
    // ancestor rows from the preorder: j is a strict ancestor of r exactly when
    // pos(j) < pos(r) <= last(pos(j)), and only j < r can be one.  Each node's
    // (pos, last) is packed once into the free children-row scratch (nodes
    // past the tree get pos 0xffff, never below a row's position); the tree's
    // workgroups share the (row, word) pairs, one pair per thread.
    const int nparts = Hv * csplit, part = h * csplit + slice;
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
        __syncthreads();
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
    // k rows of the cached blocks into registers (1 KB unit wave + 8 r: block
    // u / 4, chunk u % 4), written to LDS once the tree's gates are summed, so
    // the loads overlap that work.  Positions clamped to n - 1.
    constexpr int KCR = KC * 4 / (NT / 64);             // units per wave
    u32x4 kcr[KCR];
#pragma unroll
    for (int r = 0; r < KCR; ++r) {
        const int u = wave + (NT / 64) * r;
        const int row = node_at(16 * (u >> 2) + ln);
        kcr[r] = *reinterpret_cast<const u32x4*>(Kb + (size_t)row * kq_row + 32 * (u & 3) + 8 * lq);
    }

    // path log-gates by synchronous pointer doubling (each node adds its
    // link's sum and jumps to the link's link); round r raises flag r % 3
    // while a node still has a link to follow and clears flag (r + 1) % 3
    // before its first barrier: two LDS-only barriers per round
    for (int rd = 0;; ++rd) {
        int nn[PER], hj[PER];
        float gj[PER];
        bool more = false;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
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
        for (int k = 0; k < PER; ++k) {
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

    // G and beta by position (through the scratch: the row buffers are free)
    {
        float* tl = reinterpret_cast<float*>(&s_yrow[0][0]);
        float* tb = tl + NP;
        for (int i = tid; i < NP; i += NT) {
            const int v = node_at(i);
            tl[i] = i < n ? s_lg[v] : 0.f;
            tb[i] = i < n ? s_beta[v] : 0.f;
        }
        __syncthreads();
        for (int i = tid; i < NP; i += NT) {
            s_lg[i] = tl[i];
            s_beta[i] = tb[i];
        }
    }
    // occupancy: tile (t, s), s < t, holds an ancestor pair exactly when a
    // position of block s has its subtree reaching row t; tile lists: the
    // diagonal, then the occupied blocks in descending order, so the blocks
    // past the LDS k cache come first and get the prefetched slots
    for (int t = tid; t < NB; t += NT) {
        unsigned long long occ = 0ull;
        for (int sb = 0; sb < t && t < nblk; ++sb)
            if (s_mlast[sb] >= 16 * t) occ |= 1ull << sb;
        s_occ[t] = occ;
        s_tcol[t][0] = (uint8_t)t;
        for (int m = 1; occ; ++m) {
            const int hb = 63 - __clzll((long long)occ);
            s_tcol[t][m] = (uint8_t)hb;
            occ &= ~(1ull << hb);
        }
    }
#pragma unroll
    for (int r = 0; r < KCR; ++r)
        *reinterpret_cast<u32x4*>(s_kc + (wave + (NT / 64) * r) * 512 + lane * 8) = kcr[r];
    __syncthreads();
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    auto row_occ = [&](int t) __attribute__((always_inline)) {
        // (readfirstlane returns a signed int: widen through uint32_t, and keep
        // only column blocks 0 .. t - 1)
        return (((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(s_occ[t] >> 32)) << 32) |
                (unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)s_occ[t])) &
               ((1ull << t) - 1ull);
    };

    if (!solver) {
        // ================= Gram waves =================
        const int gw = wave - NS;
        const int pg = gw - (NG - NCG);                 // projection column group (>= 0: this wave's)
        // the projection group's S0 rows as bf16 B / A operands
        bf16x8 sb[4];
        {
            const int col0 = cbase + 16 * max(pg, 0);
            const float* p = a.S0 + ((size_t)b * Hv + h) * kD * kD + (size_t)(col0 + ln) * kD + 8 * lq;
#pragma unroll
            for (int cs = 0; cs < 4; ++cs)
                sb[cs] = to_bf16x8(*reinterpret_cast<const float4*>(p + 32 * cs),
                                   *reinterpret_cast<const float4*>(p + 32 * cs + 4));
        }
        // k / q fragment of node block blk, column chunk cs, from global memory
        // (L2): the block's base is uniform, the lane's row / column a 32-bit
        // offset (rows clamped to n - 1)
        const uint32_t lane_col = 16u * lq;                 // bytes: 8 bf16 per lane group
        auto frag = [&](const uint16_t* base, int blk, int cs) __attribute__((always_inline)) {
            const uint32_t row = (uint32_t)node_at(16 * blk + ln);
            const uint32_t off = row * (uint32_t)(kq_row * 2) + lane_col + 64u * cs;
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                  reinterpret_cast<const char*>(base) + off));
        };
        // Gram products of tile (t, s): A = K_s K_t^T, C = K_s Q_t^T (node j of
        // block s in rows, node i of block t in columns)
        auto tile_products = [&](const bf16x8 (&kt)[4], const bf16x8 (&qt)[4], const bf16x8 (&ks)[4],
                                 f32x4& A, f32x4& C) __attribute__((always_inline)) {
            A = z;
            C = z;
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
                A = mfma32(ks[cs], kt[cs], A);
                C = mfma32(ks[cs], qt[cs], C);
            }
        };
        // the products masked and decayed into -X / Y (bf16, tile layout) in the
        // row buffers of parity t & 1; for s == t the diagonal X block in fp32,
        // transposed, for the inversion
        auto tile_store = [&](int t, int s, f32x4 A, f32x4 C) __attribute__((always_inline)) {
            const int par = t & 1;
            const int i = 16 * t + ln, j0 = 16 * s + 4 * lq;
            const uint2 lw = *reinterpret_cast<const uint2*>(&s_last[j0]);     // last(j0 .. j0 + 3)
            const int lst[4] = {(int)(int16_t)(lw.x & 0xffffu), (int)(int16_t)(lw.x >> 16),
                                (int)(int16_t)(lw.y & 0xffffu), (int)(int16_t)(lw.y >> 16)};
            uint32_t bits = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) bits |= (i < n && j0 + e < i && i <= lst[e]) ? 1u << e : 0u;
            const float lgi = s_lg[i], bei = s_beta[i];
            const float4 lgj = *reinterpret_cast<const float4*>(&s_lg[j0]);
            const float lj[4] = {lgj.x, lgj.y, lgj.z, lgj.w};
            float xv[4];
            uint16_t yv[4], nxv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool anc = (bits >> e) & 1u;
                const bool self = (j0 + e == i) && i < n;
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
#pragma unroll
                for (int e = 0; e < 4; ++e) s_xd[par][(4 * lq + e) * 16 + ln] = xv[e];   // [col][row]
            }
        };
        // D = (I + X_tt)^-1 in fp32 by right-looking substitution, four lanes
        // per column: lane 4c + q holds rows 4q .. 4q+3 of column c; step m
        // broadcasts y_m from its owner within the lane quad and updates the
        // rows below it
        auto diag_inverse = [&](int t) __attribute__((always_inline)) {
            const int par = t & 1;
            const int c = lane >> 2, qd = lane & 3;
            float acc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = (4 * qd + e == c) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                const float4 xc = *reinterpret_cast<const float4*>(&s_xd[par][m * 16 + 4 * qd]);
                const float ym = quad_bcast(acc[m & 3], m >> 2);
                const float xr[4] = {xc.x, xc.y, xc.z, xc.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {                     // rows below m only
                    const float upd = fmaf(-xr[e], ym, acc[e]);
                    acc[e] = 4 * qd + e > m ? upd : acc[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) s_dinv[par][a32_pos(4 * qd + e, c)] = bf16_rne(acc[e]);
        };
        // Row t's tiles: the diagonal tile first, then the occupied column
        // blocks s < t, descending; Gram wave gw computes tiles gw, gw + NG, ...
        auto tile_col = [&](int t, unsigned long long occ, int m) __attribute__((always_inline)) {
            (void)occ;
            return __builtin_amdgcn_readfirstlane((int)s_tcol[t][m]);
        };
        // k / q fragments of a row (two sets, alternating by row) and, refilled
        // once their products are issued, the k rows of this wave's first TPW
        // tiles of the next row
        struct RowOps {
            bf16x8 k[4], q[4];
        };
        bf16x8 kp[TPW][4];
        auto load_kq = [&](RowOps& o, int t) __attribute__((always_inline)) {
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
                o.k[cs] = frag(Kb, t, cs);
                o.q[cs] = frag(Qb, t, cs);
            }
        };
        // (blocks past the LDS cache only: a cached block's slot issues no
        // load, and its products read the LDS copy)
        auto load_tile = [&](int i, int t, unsigned long long occ, int ntile) __attribute__((always_inline)) {
            const int m = gw + i * NG;
            const int sc = m < ntile ? tile_col(t, occ, m) : t;
            if constexpr (!KALL) {
                if (sc >= KC) {                             // (uniform) cached blocks read LDS instead
#pragma unroll
                    for (int cs = 0; cs < 4; ++cs) kp[i][cs] = frag(Kb, sc, cs);
                }
            } else {
                (void)sc;
            }
        };
        auto kc_frag = [&](int sblk, int cs) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8*>(s_kc + (min(sblk, KC - 1) * 4 + cs) * 512 + lane * 8);
        };
        // step t: row t + 1's tiles and projections (operands in cur, its first
        // tiles' k rows in kp), requesting row t + 2's operands into nxt and kp;
        // the last rows re-read the last row (harmless).  The first TPW tiles'
        // products are issued together (independent chains), then their k
        // registers are refilled, then they are masked and stored.
        auto gstep = [&](int t, const RowOps& cur, RowOps& nxt) __attribute__((always_inline)) {
            if (t + 1 < nblk) {
                const int tr = t + 1, tn = min(t + 2, nblk - 1);
                load_kq(nxt, tn);
                const unsigned long long occ = row_occ(tr), occn = row_occ(tn);
                const int ntile = __popcll(occ) + 1, ntn = __popcll(occn) + 1;
                f32x4 Ap[TPW], Cp[TPW];
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    const int m = gw + i * NG;
                    const int sc = m < ntile ? tile_col(tr, occ, m) : tr;    // (unused slot: a valid tile)
                    bf16x8 ks[4];
#pragma unroll
                    for (int cs = 0; cs < 4; ++cs) {
                        if constexpr (KALL) ks[cs] = kc_frag(sc, cs);
                        else ks[cs] = sc < KC ? kc_frag(sc, cs) : kp[i][cs];
                    }
                    tile_products(cur.k, cur.q, ks, Ap[i], Cp[i]);
                }
#pragma unroll
                for (int i = 0; i < TPW; ++i) load_tile(i, tn, occn, ntn);
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    const int m = gw + i * NG;
                    if (m < ntile) tile_store(tr, tile_col(tr, occ, m), Ap[i], Cp[i]);
                }
                for (int m = gw + TPW * NG; m < ntile; m += NG) {
                    const int sc = tile_col(tr, occ, m);
                    bf16x8 k0[4];
#pragma unroll
                    for (int cs = 0; cs < 4; ++cs) k0[cs] = sc < KC ? kc_frag(sc, cs) : frag(Kb, sc, cs);
                    f32x4 A0, C0;
                    tile_products(cur.k, cur.q, k0, A0, C0);
                    tile_store(tr, sc, A0, C0);
                }
                // projections of row t + 1 for column group pg
                if (pg >= 0) {
                    f32x4 pk = z, pq = z;
#pragma unroll
                    for (int cs = 0; cs < 4; ++cs) {
                        pk = mfma32(cur.k[cs], sb[cs], pk);     // [node][r]
                        pq = mfma32(sb[cs], cur.q[cs], pq);     // [r][node]
                    }
                    s_pk[tr & 1][pg][lane] = pk;
                    s_pq[tr & 1][pg][lane] = pq;
                }
                if (gw == 0) diag_inverse(tr);                  // the diagonal tile is this wave's first
            }
            lds_barrier();
        };
        RowOps A, B;
        load_kq(A, 0);
        {
            const unsigned long long occ0 = row_occ(0);
#pragma unroll
            for (int i = 0; i < TPW; ++i) load_tile(i, 0, occ0, __popcll(occ0) + 1);
        }
        gstep(-1, A, B);                                // row 0; requests row 1
        for (int t = 0; t < nblk; t += 2) {
            gstep(t, B, A);
            if (t + 1 < nblk) gstep(t + 1, A, B);
        }
        return;
    }

    // ================= solve waves =================
    const int c0 = cbase + 16 * CG * wave;              // this wave's first value column
    const s16x4 zero4 = {0, 0, 0, 0};
    const bool hi_half = lq >= 2;
    s16x4 ident;
#pragma unroll
    for (int e = 0; e < 4; ++e) ident[e] = (4 * lq + e == ln) ? (short)0x3f80 : (short)0;
    bf16x8 up[CG][NPR];                                 // [U_2p; U_2p+1] as 16x16x32 B operands
#pragma unroll
    for (int g = 0; g < CG; ++g)
#pragma unroll
        for (int p = 0; p < NPR; ++p) up[g][p] = zero8;

    // row t of the blocked substitution and the output stage for this wave's
    // two column groups, from the published tiles and projections of row t
    // (parity t & 1); every tile read feeds both groups
    auto solve_row = [&](int t, const uint2 (&vt)[CG]) __attribute__((always_inline)) {
        const int par = t & 1;
        const unsigned long long occ = row_occ(t);
        const uint16_t* xr = s_xrow[par];
        const uint16_t* yr = s_yrow[par];
        f32x4 R[CG], pqT[CG];
#pragma unroll
        for (int g = 0; g < CG; ++g) {
            const f32x4 pk = s_pk[par][CG * wave + g][lane];
            pqT[g] = s_pq[par][CG * wave + g][lane];
            const f32x4 vd = mfma16(__builtin_bit_cast(s16x4, vt[g]), ident, z);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int i = 16 * t + 4 * lq + m;
                R[g][m] = s_beta[i] * (vd[m] - __expf(s_lg[i]) * pk[m]);
            }
        }
        // R_t += sum_{s<t} (-X_ts) U_s over occupied tiles, two blocks per MFMA;
        // even and odd pairs accumulate apart (four independent chains)
        f32x4 R2[CG];
#pragma unroll
        for (int g = 0; g < CG; ++g) R2[g] = z;
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
            const int s = 2 * p;
            if (s < t) {
                const bool o0 = (occ >> s) & 1ull;
                const bool o1 = s + 1 < t && ((occ >> (s + 1)) & 1ull);
                if (o0 || o1) {
                    bf16x8 nx = *reinterpret_cast<const bf16x8*>(xr + s * 256 + lane * 8);
                    if (!(hi_half ? o1 : o0)) nx = zero8;
#pragma unroll
                    for (int g = 0; g < CG; ++g) {
                        if (p & 1) R2[g] = mfma32(nx, up[g][p], R2[g]);
                        else R[g] = mfma32(nx, up[g][p], R[g]);
                    }
                }
            }
        }
#pragma unroll
        for (int g = 0; g < CG; ++g) R[g] += R2[g];
        const bf16x8 di = *reinterpret_cast<const bf16x8*>(s_dinv[par] + (ln + 16 * (lq & 1)) * 8);
        const int node = 16 * t + ln;
#pragma unroll
        for (int g = 0; g < CG; ++g) {
            s16x4 rh, rl;
            split4(R[g], rh, rl);
            const bf16x8 rr = stack_pair(rh, rl);
            const f32x4 U = mfma32(di, rr, z);
            const f32x4 UT = mfma32(rr, di, z);
            const s16x4 ut = to_bf16x4(U);
#pragma unroll
            for (int p = 0; p < NPR; ++p) {
                if (p == (t >> 1)) {
                    if (t & 1)
                        up[g][p] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, up[g][p]) |
                                                                  __builtin_bit_cast(u32x4, stack_pair(zero4, ut)));
                    else
                        up[g][p] = stack_pair(ut, zero4);
                }
            }
            if (node < n) *reinterpret_cast<f32x4*>(Ug + (size_t)node_at(node) * kD + c0 + 16 * g + 4 * lq) = UT;
        }
        // O_t^T = e^G P_Q^T + sum_{s<=t} U_s^T Y_ts^T over occupied tiles
        f32x4 Oc[CG], Oc2[CG];
#pragma unroll
        for (int g = 0; g < CG; ++g) Oc[g] = Oc2[g] = z;
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
            const int s = 2 * p;
            if (s <= t) {
                const bool o0 = s == t || ((occ >> s) & 1ull);
                const bool o1 = s + 1 == t || (s + 1 < t && ((occ >> (s + 1)) & 1ull));
                if (o0 || o1) {
                    bf16x8 yt = *reinterpret_cast<const bf16x8*>(yr + s * 256 + lane * 8);
                    if (!(hi_half ? o1 : o0)) yt = zero8;
#pragma unroll
                    for (int g = 0; g < CG; ++g) {
                        if (p & 1) Oc2[g] = mfma32(up[g][p], yt, Oc2[g]);
                        else Oc[g] = mfma32(up[g][p], yt, Oc[g]);
                    }
                }
            }
        }
#pragma unroll
        for (int g = 0; g < CG; ++g) Oc[g] += Oc2[g];
        if (node < n) {
            const float egn = __expf(s_lg[node]);
#pragma unroll
            for (int g = 0; g < CG; ++g) {
                f32x4 OT;
#pragma unroll
                for (int m = 0; m < 4; ++m) OT[m] = egn * pqT[g][m] + Oc[g][m];
                const uint32_t lo = (uint32_t)bf16_rne(OT[0]) | ((uint32_t)bf16_rne(OT[1]) << 16);
                const uint32_t hi = (uint32_t)bf16_rne(OT[2]) | ((uint32_t)bf16_rne(OT[3]) << 16);
                *reinterpret_cast<uint2*>(O + vo_base + (size_t)node_at(node) * vo_row + c0 + 16 * g + 4 * lq) =
                    make_uint2(lo, hi);
            }
        }
    };
    // v of row t + 1 is requested before row t's stores (loads and stores
    // retire in order, so waiting for it never waits for those stores)
    const uint16_t* Vp = static_cast<const uint16_t*>(a.v) + vo_base + c0 + 4 * lq;
    auto load_v = [&](int t, uint2 (&v)[CG]) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < CG; ++g)
            v[g] = *reinterpret_cast<const uint2*>(Vp + (size_t)node_at(16 * t + ln) * vo_row + 16 * g);
    };
    uint2 va[CG], vb[CG];
    load_v(0, va);
    lds_barrier();
    for (int t = 0; t < nblk; t += 2) {
        load_v(min(t + 1, nblk - 1), vb);
        solve_row(t, va);
        lds_barrier();
        if (t + 1 < nblk) {
            load_v(min(t + 2, nblk - 1), va);
            solve_row(t + 1, vb);
            lds_barrier();
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
    // two column slices of 64 value columns per (sequence, value head), eight
    // waves each: two solve waves of 32 columns (trees up to 256 nodes) or four
    // of 16 (up to 512), each holding 16 stacked U pairs, one wave per SIMD
    int csplit = 2;
    const void* fn = a.N <= 256 ? (const void*)verify_large_kernel<16> : (const void*)verify_large_kernel<32>;
    void* args[] = {&copy, &csplit};
    return hipLaunchKernel(fn, dim3((unsigned)(a.B * a.Hv * csplit)), dim3(512), args, 0, stream);
}

}  // namespace gdn
