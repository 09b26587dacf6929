// verify_tiled.hip -- MFMA tree verification for d_k = d_v = 128, bf16 q/k/v/o
// and trees of up to 16 * NB nodes (NB = 4 or 8 blocks of 16 nodes).
//
// Method (page "Trees from Marginals: Autoregressive drafting with factorized
// priors", section 3, rollback-free tree verification for GDN): with G_i the
// path sum of ln g and the ancestor relation of the topologically sorted tree,
//     X_ij = beta_i e^(G_i-G_j) k_i.k_j  (j strict ancestor of i), else 0
//     Y_ij = e^(G_i-G_j) q_i.k_j         (j ancestor of i, or j = i), else 0
//     (I + X) U = R,  R = diag(beta) (V - diag(e^G) K S0^T)
//     O = diag(e^G) Q S0^T + Y U.
// The section names the three fused stages this kernel runs in one pass: the
// Gram matrix, a tiled forward substitution, and the output stage.
//
// Persistent workgroups (one per CU) loop over work items = (sequence, key
// head, group of HPW value heads); four waves per value head, each owning 32
// value columns as two interleaved 16-column groups.  Per item:
//  1. one wave builds the tree's strict-ancestor bit rows and the path
//     log-gates G by synchronous pointer doubling in LDS;
//  2. Gram tiles K_s K_t^T and K_s Q_t^T (16 x 16, s <= t) on
//     v_mfma_f32_16x16x32_bf16, shared by the HPW heads, masked and decayed per
//     head into bf16 -X / Y tiles (stored as halves of 16x16x32 A operands)
//     and fp32 diagonal X blocks;
//  3. each diagonal block (I + X_tt) is inverted in fp32;
//  4. each wave runs its columns through the blocked substitution and the
//     output stage with no barrier, two node blocks per MFMA.
// The next item's inputs load while this one computes (details at the kernel).
//
// HBM traffic is the algorithm's own: S0 once (fp32, rounded to bf16 on
// chip), k / q once per item, v once, o (bf16) and the u / G cache (fp32)
// written once.  Nothing writes S0.
#include "gdn_common.hpp"
#include "launch.hpp"
#include "mfma_tiles.hpp"

namespace gdn {

namespace {

// 16-byte chunk (row, chunk) of a k / q row in LDS; chunks are XOR-swizzled by
// the row's low bits so the 16 rows of a fragment read hit distinct banks.
__device__ __forceinline__ int kq_off(int row, int chunk) {
    return row * kD + ((chunk ^ (row & 15)) << 3);
}

// A/B fragment of a 16-node block for the 16x16x32 MFMA from LDS: lane l gets
// row 16*blk + l%16, columns 32*cs + 8*(l/16) .. +7.
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* m, int blk, int cs, int lane) {
    const int row = 16 * blk + (lane & 15);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                          m + kq_off(row, 4 * cs + (lane >> 4))));
}

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Persistent workgroups, one per CU (two per CU for one-head workgroups on
// trees of up to 64 nodes, whose register budget is capped at 256 per lane for
// that), each looping over (sequence, key head, head group) work items with the
// next item's inputs in flight:
//  - at the start of item n's solve (before its output stores, since loads
//    and stores retire in order): item n+1's parent / g / beta words and S0
//    rows into registers;
//  - once item n's solve is done with k / q: item n+1's k / q rows straight
//    from HBM into LDS (global_load_lds);
//  - item n+1's v rows after its tree, used only after its Gram.
// One explicit wait per item (its k / q / S0 landed) before the Gram, one
// (its v landed) before the solve; the solve itself never waits on memory.
//
// Waves: four per value head; wave (hp, wc) owns value columns 32 wc .. +31 of
// head h0 + hp as two 16-column groups, so every k / q / tile fragment it
// reads from LDS feeds two MFMA chains.
// FUSED: the kernel first commits the previous tree's accepted node (args c;
// its state is this launch's S0, a.S0 = c.S_in) into the S0 rows each wave
// holds, writes them to c.S_out and verifies with them (see the commit prologue).
// RAGGED: per-node arrays in the ragged layout (a.offsets, and c.offsets for
// the previous tree); a tree of n < N nodes runs only its ceil(n / 16) blocks.
// Loads never leave a tree's rows: rows past n re-read row n - 1, and an empty
// tree's loads read the first line of S0 instead.
template <int NB, int HPW, bool FUSED, bool RAGGED>
__global__ __launch_bounds__(256 * HPW, HPW == 1 && NB == 4 ? 2 : 1) void verify_tiled_kernel(VerifyArgs a, CommitArgs c, int nitems) {
    constexpr int WPH = 4;                      // waves per value head
    constexpr int CG = 2;                       // 16-column groups per wave
    constexpr int NW = WPH * HPW;               // waves
    constexpr int NT = 64 * NW;                 // threads
    constexpr int NP = 16 * NB;                 // padded node count
    constexpr int NX = NB * (NB - 1) / 2;       // strictly-lower X tiles
    constexpr int NPAIR = NB * (NB + 1) / 2;    // Gram tiles (s <= t)
    constexpr int MW = NP / 32 > 0 ? NP / 32 : 1;
    constexpr int KQ_INS = 2 * NP / 4;          // 1 KB direct-to-LDS loads for k and q
    constexpr int NPL = NP / 64;                // nodes per lane of the tree wave
    static_assert(NPL >= 1 && NT >= 64 + NP, "tree wave plus beta threads");
    static_assert(KQ_INS % NW == 0, "whole direct-to-LDS loads per wave");
    __shared__ __attribute__((aligned(16))) uint16_t s_k[NP * kD];
    __shared__ __attribute__((aligned(16))) uint16_t s_q[NP * kD];
    // -X then Y tiles; one spare tile at the end: a row's last pair may read
    // 512 bytes past its last tile (those lanes are zeroed before use)
    __shared__ __attribute__((aligned(16))) uint16_t s_tiles[HPW][NB * NB * 256 + 256];
    __shared__ __attribute__((aligned(16))) uint16_t s_dinv[HPW][NB * 256];
    __shared__ __attribute__((aligned(16))) float s_xd[HPW][NB * 256];
    __shared__ __attribute__((aligned(16))) uint32_t s_mask[NP * MW];
    __shared__ __attribute__((aligned(16))) int32_t s_jump[NP];
    __shared__ __attribute__((aligned(16))) float s_lg[HPW][NP];
    __shared__ __attribute__((aligned(16))) float s_beta[HPW][NP];
    __shared__ int s_flag;

    const int N = a.N, Hv = a.Hv, Hk = a.Hk, G = Hv / Hk, GG = G / HPW;
    const int W = (N + 31) / 32;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hp = wave / WPH, wc = wave % WPH;       // this wave: head h0+hp, cols 32wc..
    const int col0 = 32 * wc;
    const size_t vo_row = (size_t)Hv * kD;            // stride between nodes in v / o
    // Thread index, re-read through an empty asm at every item so that the many
    // thread-derived LDS / global addresses are recomputed per item instead of
    // being hoisted out of the item loop (which would pin them in registers).
    int tid = threadIdx.x;
    int lane = tid & 63;
    int ln = lane & 15, lq = lane >> 4;

    // work slot -> (sequence, key head, head group).  Slot it runs on workgroup
    // it % grid in round it / grid; workgroups are dealt to the eight XCDs
    // round robin, so within a full round the slots are renumbered XCD by XCD:
    // the grid / 8 workgroups of one XCD take consecutive items, and the items
    // of one sequence (which share its parent row and the g / beta lines) meet
    // in one L2.
    const int grid = gridDim.x;
    auto decode = [&](int it, int& b, int& hk, int& hg) {
        const int r = it / grid, x = it - r * grid;
        if ((grid & 7) == 0 && (r + 1) * grid <= nitems) it = r * grid + (x & 7) * (grid >> 3) + (x >> 3);
        hg = it % GG;
        const int bh = it / GG;
        hk = bh % Hk;
        b = bh / Hk;
    };
    // rows of sequence b in the node arrays (dense: b N .., N nodes)
    auto tree_rows = [&](const int32_t* offsets, int b) {
        if constexpr (RAGGED) return seq_rows(offsets, b, N);
        else return SeqRows{(int64_t)b * N, N};
    };
    // the current item's tree: node count (0 for unusable offsets) and whether
    // its offsets are unusable
    int tn = N;
    bool tbad = false;

    // ---- prefetch helpers (registers / LDS written by loads in flight) ----
    // Per item, wave 0 needs parent and g of nodes lane + 64k (k < NPL), and the
    // threads 64 .. 64 + NP - 1 need beta of node tid - 64; every thread issues
    // the same number of loads into the same registers (addresses chosen per
    // wave, indices clamped), so no load sits under a branch: a load under a
    // branch would leave a control-flow merge that copies its result, and the
    // copy would wait for every older load and store of the wave.
    constexpr int NSM = NPL * (1 + HPW);
    uint32_t sm[NSM];
    // (real = false: a placeholder after the last item, every lane reading one
    // word, so that the loads still happen but move next to no bytes)
    auto load_small = [&](int it, bool real) {
        int b, hk, hg;
        decode(it, b, hk, hg);
        const int h0 = hk * G + hg * HPW;
        const SeqRows rw = tree_rows(a.offsets, b);
        if (RAGGED && rw.n <= 0) real = false;
        const uint32_t* par = reinterpret_cast<const uint32_t*>(a.parent) + rw.row0;
        const uint32_t* gg = reinterpret_cast<const uint32_t*>(wave == 0 ? a.g : a.beta) +
                             rw.row0 * Hv + h0;
        if (RAGGED && !real) par = gg = reinterpret_cast<const uint32_t*>(a.S0);
        const int nb = real ? min(max(tid - 64, 0), rw.n - 1) : 0;
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const int i = real ? min(lane + 64 * k, rw.n - 1) : 0;
            sm[k] = par[i];
#pragma unroll
            for (int p = 0; p < HPW; ++p)
                sm[NPL + k * HPW + p] = gg[(size_t)(wave == 0 ? i : nb) * Hv + p];
        }
    };
    // k and q rows of the item's tree into s_k / s_q: each wave instruction
    // fills 1 KB (4 rows) of LDS, lane l landing on row r0 + l/16, physical chunk
    // l%16, which holds logical chunk (l%16) ^ (row & 15).  Rows past the tree's
    // n copy row n - 1 (finite values; masks and beta = 0 keep them out of every
    // result).
    // (real = false: a placeholder after the last item, every lane reading one line)
    auto kq_dma = [&](int it, bool real) {
        int b, hk, hg;
        decode(it, b, hk, hg);
        const SeqRows rw = tree_rows(a.offsets, b);
        if (RAGGED && rw.n <= 0) real = false;
        const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + (rw.row0 * Hk + hk) * kD;
        const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + (rw.row0 * Hk + hk) * kD;
        if (RAGGED && !real) Kb = reinterpret_cast<const uint16_t*>(a.S0);
#pragma unroll
        for (int kk = 0; kk < KQ_INS / NW; ++kk) {      // compile-time count: a loop of
            const int ins = wave + kk * NW;            // loads would get a full wait ahead
            const int mat = ins / (NP / 4), r0 = (ins % (NP / 4)) * 4;
            const int row = r0 + (lane >> 4), pc = lane & 15;
            const int srow = row < rw.n ? row : rw.n - 1;
            const uint16_t* src = real ? (mat ? Qb : Kb) + (size_t)srow * Hk * kD + ((pc ^ (row & 15)) << 3) : Kb;
            uint16_t* dst = (mat ? s_q : s_k) + r0 * kD;
            __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)dst, 16, 0, 0);
        }
    };
    float4 s0raw[CG][4][2];
    // this wave's S0 rows of column group g, key columns 32c + 8(l/16)..+7.
    // Group g's local row rho is value column col0 + 8 (rho / 4) + 4g + rho % 4:
    // the groups interleave in runs of 4, so the 4 + 4 values a lane holds for
    // one node in the transposed outputs (and the v values it needs) are 8
    // consecutive columns, one 16-byte access for both groups.
    // (real = false: the placeholder loads of the last item, all from one line)
    auto load_s0 = [&](int it, int g, bool real) {
        int b, hk, hg;
        decode(it, b, hk, hg);
        const int h = hk * G + hg * HPW + hp;
        const int row = col0 + 8 * (ln >> 2) + 4 * g + (ln & 3);
        const float* p0 = a.S0 + ((size_t)b * Hv + h) * kD * kD + (size_t)row * kD + 8 * lq;
        const int cstep = real ? 32 : 0;
        if (!real) p0 = a.S0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s0raw[g][c][0] = *reinterpret_cast<const float4*>(p0 + cstep * c);
            s0raw[g][c][1] = *reinterpret_cast<const float4*>(p0 + cstep * c + (real ? 4 : 0));
        }
    };

    // The item's tree, built by wave 0 alone, with no workgroup barrier, by
    // synchronous pointer doubling.  Lane l owns nodes l + 64k.  Node i keeps a
    // covered set C_i (itself and its nearest ancestors, a bit row), the sums of
    // ln g over C_i for each value head, and nx_i, its nearest ancestor outside
    // C_i (-1 once C_i reaches the root).  A round adds C_(nx_i) and its sums
    // and moves nx_i to nx_(nx_i); all lanes finish reading before any lane
    // writes, so a round sees only the previous round's values and C_i doubles:
    // ceil(log2(depth)) + 1 rounds.  Then C_i is i with all its ancestors and
    // the sums are the path log-gates G_i.  Leaves the strict-ancestor rows in
    // s_mask (row stride MW), G in s_lg and the tree status in s_flag.
    auto tree_wave = [&]() {
        int status = 0;
#pragma unroll
        for (int k = NPL - 1; k >= 0; --k) {                // lowest bad node wins
            const int i = lane + 64 * k, pi = (int)sm[k];
            const uint64_t bad = __ballot(i < tn && (pi < -1 || pi >= i));
            if (bad) status = 64 * k + __ffsll((unsigned long long)bad);
        }
        if (tbad) status = -1;
        int nx[NPL];
        uint32_t m[NPL][MW];
        float gv[NPL][HPW];
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const int i = lane + 64 * k;
            const bool valid = i < tn && status == 0;
            nx[k] = valid ? (int)sm[k] : -1;
#pragma unroll
            for (int w = 0; w < MW; ++w) m[k][w] = (valid && (i >> 5) == w) ? 1u << (i & 31) : 0u;
#pragma unroll
            for (int p = 0; p < HPW; ++p)
                gv[k][p] = valid ? logf(__uint_as_float(sm[NPL + k * HPW + p])) : 0.f;
            s_jump[i] = nx[k];
#pragma unroll
            for (int w = 0; w < MW; ++w) s_mask[i * MW + w] = m[k][w];
#pragma unroll
            for (int p = 0; p < HPW; ++p) s_lg[p][i] = gv[k][p];
        }
        for (;;) {
            bool act = false;
#pragma unroll
            for (int k = 0; k < NPL; ++k) act |= nx[k] >= 0;
            if (!__any(act)) break;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // last round's writes done
            int nn[NPL];
            uint32_t mj[NPL][MW];
            float gj[NPL][HPW];
#pragma unroll
            for (int k = 0; k < NPL; ++k) {
                const int j = nx[k] >= 0 ? nx[k] : lane + 64 * k;
                nn[k] = s_jump[j];
#pragma unroll
                for (int w = 0; w < MW; ++w) mj[k][w] = s_mask[j * MW + w];
#pragma unroll
                for (int p = 0; p < HPW; ++p) gj[k][p] = s_lg[p][j];
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // every read done
#pragma unroll
            for (int k = 0; k < NPL; ++k) {
                const int i = lane + 64 * k;
                if (nx[k] >= 0) {
#pragma unroll
                    for (int w = 0; w < MW; ++w) m[k][w] |= mj[k][w];
#pragma unroll
                    for (int p = 0; p < HPW; ++p) gv[k][p] += gj[k][p];
                    nx[k] = nn[k];
                }
                s_jump[i] = nx[k];
#pragma unroll
                for (int w = 0; w < MW; ++w) s_mask[i * MW + w] = m[k][w];
#pragma unroll
                for (int p = 0; p < HPW; ++p) s_lg[p][i] = gv[k][p];
            }
        }
#pragma unroll
        for (int k = 0; k < NPL; ++k) {                     // strict-ancestor rows
            const int i = lane + 64 * k;
#pragma unroll
            for (int w = 0; w < MW; ++w)
                s_mask[i * MW + w] = (i >> 5) == w ? m[k][w] & ~(1u << (i & 31)) : m[k][w];
        }
        if (lane == 0) s_flag = status;
    };
    // The tree part of the cache, from LDS once the tree is published: ancestor
    // rows, depth and status (one head group per sequence writes them) and the
    // path log-gates of this item's value heads.
    auto write_tree_cache = [&](int b, int h0, bool writer, int status) {
        uint32_t* gm = a.anc_mask + (size_t)b * N * W;
        for (int i = lane; i < N; i += 64) {
            if (writer) {
                int cnt = 0;
#pragma unroll
                for (int w = 0; w < MW; ++w) {
                    const uint32_t x = s_mask[i * MW + w];
                    if (w < W) gm[(size_t)i * W + w] = x;
                    cnt += __popc(x);
                }
                a.depth[(size_t)b * N + i] = (status || i >= tn) ? -1 : cnt;
            }
            if (status == 0) {
#pragma unroll
                for (int p = 0; p < HPW; ++p)
                    a.log_gamma[((size_t)b * Hv + h0 + p) * N + i] = s_lg[p][i];
            }
        }
        if (writer && lane == 0) a.status[b] = status;
    };

    s16x4 ident;                                      // I as a 16x16x16 B operand
#pragma unroll
    for (int e = 0; e < 4; ++e) ident[e] = (4 * lq + e == ln) ? (short)0x3f80 : (short)0;

    // ---- commit of the previous tree (FUSED) ----------------------------------
    // Page section 3 defers the commit of the accepted node to the next step;
    // here it runs on the S0 rows each wave holds for the item (s0raw, which
    // hold S_prev): S_a = e^(G_a) S_prev + sum_{j in P} e^(G_a - G_j) u_j k_j^T
    // with G, u from the previous tree's cache and k its keys.  P is the
    // accepted node with its ancestors (its ancestor row), enumerated root
    // first: slot m < |P| - 1 is the m-th set bit of the row, the last slot the
    // accepted node.  The update is a rank-|P| product on the matrix cores:
    // per 32 path slots, D^T += K_P^T (w u_P) with K_P^T (key column x slot,
    // bf16 inputs, exact) and w u_P (slot x value row) split into bf16 hi + lo,
    // staged transposed in the tile area (free until the Gram).  D^T comes out
    // in exactly the layout s0raw holds.  The committed rows go to c.S_out and
    // become this item's S0; one item per sequence writes the previous tree's
    // path.  Latency is hidden by prefetch: the accepted node and tree status
    // load with the item's small loads one item ahead, the ancestor row at the
    // end of the item before, and the first 32 slots' k / u rows and log-gates
    // at the item's start, landing with its tree.
    constexpr int SLOT_BYTES = kD * 2 + HPW * kD * 4;           // k column, w u hi + lo
    constexpr int PC_ROOM = ((int)sizeof(s_tiles) - NW * NP * 4) / SLOT_BYTES;
    constexpr int PC = PC_ROOM >= 32 ? 32 : PC_ROOM >= 16 ? 16 : 8;
    static_assert(PC * SLOT_BYTES <= (int)sizeof(s_tiles), "path staging fits the tile area");
    constexpr int KR = FUSED ? (PC * 16 + NT - 1) / NT : 0;     // k loads per thread
    constexpr int UR = FUSED ? (HPW * PC * 32 + NT - 1) / NT : 0;   // u loads per thread
    int cm_acc_v = 0, cm_st_v = 0;              // loads in flight
    int cm_acc = 0, cm_st = 0;                  // the same, uniform
    SeqRows prv{0, N};                          // this item: the previous tree's rows
    uint32_t cm_row_v[MW];
#pragma unroll
    for (int w = 0; w < MW; ++w) cm_row_v[w] = 0u;
    uint32_t pw[MW];                            // this item: path row (uniform)
    int plen = -1;                              // |P|; 0 nothing accepted, -1 no commit
    u32x4 st_k[KR > 0 ? KR : 1];
    float4 st_u[UR > 0 ? UR : 1];
    float st_lj[UR > 0 ? UR : 1];
    float st_la[HPW];
    // staging, transposed: kT[kk][slot], wh / wl[head][value row][slot]; slots
    // past the path are zero.  After it, each wave's slot -> node table.
    uint16_t* const kT = reinterpret_cast<uint16_t*>(&s_tiles[0][0]);
    uint16_t* const wh = kT + kD * PC;
    uint16_t* const wl = wh + HPW * kD * PC;
    int* const ptab = reinterpret_cast<int*>(wl + HPW * kD * PC) + wave * NP;
    static_assert(PC * SLOT_BYTES + NW * NP * 4 <= (int)sizeof(s_tiles), "slot tables fit");
    static_assert(MW == 2 * NPL && NP % PC == 0, "word / lane split of the path row");
    auto commit_small = [&](int it) {
        int b, hk, hg;
        decode(it, b, hk, hg);
        cm_acc_v = c.accepted[b];
        cm_st_v = c.status[b];
    };
    auto commit_take_small = [&]() {
        cm_acc = __builtin_amdgcn_readfirstlane(cm_acc_v);
        cm_st = __builtin_amdgcn_readfirstlane(cm_st_v);
    };
    auto commit_row = [&](int it) {
        int b, hk, hg;
        decode(it, b, hk, hg);
        const uint32_t* prow = c.anc_mask + ((size_t)b * N + min(max(cm_acc, 0), N - 1)) * W;
#pragma unroll
        for (int w = 0; w < MW; ++w) cm_row_v[w] = prow[min(w, W - 1)];
    };
    auto commit_path = [&]() {
        const bool valid = cm_st == 0 && cm_acc >= -1 && cm_acc < prv.n;
        int pc = 0;
#pragma unroll
        for (int w = 0; w < MW; ++w) {
            const uint32_t x = (uint32_t)__builtin_amdgcn_readfirstlane((int)cm_row_v[w]);
            pw[w] = (w < W && valid && cm_acc >= 0) ? x : 0u;
            pc += __popc(pw[w]);
        }
        plen = valid ? (cm_acc < 0 ? 0 : pc + 1) : -1;
        // slot -> node table, one private copy per wave: lane l tests nodes
        // l + 64k, a set bit's slot is its rank among the set bits
        int base = 0;
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const uint32_t word = lane < 32 ? pw[2 * k] : pw[2 * k + 1];
            const bool on = (word >> (lane & 31)) & 1u;
            const uint64_t bal = __ballot(on);
            const int rank = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (on) ptab[rank] = lane + 64 * k;
            base += __popcll(bal);
        }
        asm volatile("" ::: "memory");
    };
    // node of path slot s (s < plen); other slots: the accepted node (clamped),
    // so that every load stays in bounds and padding rereads a cached row
    auto slot_node = [&](int s) {
        const int last = min(max(cm_acc, 0), N - 1);
        const int t = ptab[s];                          // s < NP: always in the table
        return s < plen - 1 ? min(t, N - 1) : last;
    };
    auto commit_issue = [&](int b, int hk, int h0, int p0) {
        const uint16_t* Kp = static_cast<const uint16_t*>(c.k) + prv.row0 * Hk * kD + hk * kD;
        // (path nodes lie below the accepted node; padding slots re-read its
        // row, or, with nothing in the previous tree, the first line of S_in)
        const int klast = RAGGED ? max(prv.n - 1, 0) : N - 1;
        if (RAGGED && prv.n <= 0) Kp = reinterpret_cast<const uint16_t*>(c.S_in);
        const float* Up = c.u + ((size_t)b * Hv + h0) * (size_t)N * kD;
        const float* lgprev = c.log_gamma + ((size_t)b * Hv + h0) * N;
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const int x = min(tid + r * NT, PC * 16 - 1);
            const int m = x % PC, ck = x / PC;
            const int j = min(slot_node(p0 + m), klast);
            st_k[r] = *reinterpret_cast<const u32x4*>(Kp + (size_t)j * Hk * kD + 8 * ck);
        }
#pragma unroll
        for (int r = 0; r < UR; ++r) {
            const int x = min(tid + r * NT, HPW * PC * 32 - 1);
            const int m = x % PC, f = (x / PC) % 32, p = x / (PC * 32);
            const int j = slot_node(p0 + m);
            st_u[r] = *reinterpret_cast<const float4*>(Up + ((size_t)p * N + j) * kD + 4 * f);
            st_lj[r] = lgprev[(size_t)p * N + j];
        }
        const int ja = min(max(cm_acc, 0), N - 1);
#pragma unroll
        for (int p = 0; p < HPW; ++p) st_la[p] = lgprev[(size_t)p * N + ja];
    };
    auto commit_stage = [&](int p0) {
        const int pn = plen - p0;
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const int x = tid + r * NT;
            if (PC * 16 % NT == 0 || x < PC * 16) {
                const int m = x % PC, ck = x / PC;
                const u32x4 kv = m < pn ? st_k[r] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kT[(8 * ck + 2 * e) * PC + m] = (uint16_t)(kv[e] & 0xffffu);
                    kT[(8 * ck + 2 * e + 1) * PC + m] = (uint16_t)(kv[e] >> 16);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < UR; ++r) {
            const int x = tid + r * NT;
            if (HPW * PC * 32 % NT == 0 || x < HPW * PC * 32) {
                const int m = x % PC, f = (x / PC) % 32, p = x / (PC * 32);
                const float wgt = __expf(st_la[p] - st_lj[r]);
                const float uu[4] = {st_u[r].x, st_u[r].y, st_u[r].z, st_u[r].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float val = m < pn ? wgt * uu[i] : 0.f;
                    const uint16_t hi = bf16_rne(val);
                    const int at = (p * kD + 4 * f + i) * PC + m;
                    wh[at] = hi;
                    wl[at] = bf16_rne(val - bf16_val(hi));
                }
            }
        }
    };
    auto commit_apply = [&](int b, int hk, int hg, int h0, int h) {
        if (hk == 0 && hg == 0) {
            for (int m = tid; m < prv.n; m += NT) c.path[prv.row0 + m] = m < plen ? slot_node(m) : -1;
            if (tid == 0) c.path_len[b] = plen;
        }
        if (plen > 0) {
            const float dec = __expf(st_la[hp]);
#pragma unroll
            for (int g = 0; g < CG; ++g)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2) {
                        s0raw[g][cc][q2].x *= dec; s0raw[g][cc][q2].y *= dec;
                        s0raw[g][cc][q2].z *= dec; s0raw[g][cc][q2].w *= dec;
                    }
            const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
            const bool lane_on = 8 * lq < PC;               // K = 32 operand lanes past PC slots: 0
            const int lqs = lane_on ? lq : 0;
            for (int p0 = 0;;) {
                bf16x8 bh[CG], bl[CG];
#pragma unroll
                for (int g = 0; g < CG; ++g) {
                    const int row = col0 + 8 * (ln >> 2) + 4 * g + (ln & 3);
                    const int at = (hp * kD + row) * PC + 8 * lqs;
                    bh[g] = lane_on ? *reinterpret_cast<const bf16x8*>(wh + at) : zero8;
                    bl[g] = lane_on ? *reinterpret_cast<const bf16x8*>(wl + at) : zero8;
                }
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2) {
                        const int kk = 32 * cc + 8 * (ln >> 2) + 4 * q2 + (ln & 3);
                        const bf16x8 ak = lane_on ? *reinterpret_cast<const bf16x8*>(kT + kk * PC + 8 * lqs) : zero8;
#pragma unroll
                        for (int g = 0; g < CG; ++g) {
                            f32x4 d = __builtin_bit_cast(f32x4, s0raw[g][cc][q2]);
                            d = mfma32(ak, bh[g], d);
                            d = mfma32(ak, bl[g], d);
                            s0raw[g][cc][q2] = __builtin_bit_cast(float4, d);
                        }
                    }
                p0 += PC;
                lds_barrier();                              // staging read by every wave
                if (p0 >= plen) break;
                commit_issue(b, hk, h0, p0);
                wait_vmem_all();
                commit_stage(p0);
                lds_barrier();
            }
        }
        // this wave's rows of the committed state, where S0 was read from
#pragma unroll
        for (int g = 0; g < CG; ++g) {
            const int row = col0 + 8 * (ln >> 2) + 4 * g + (ln & 3);
            float* p = c.S_out + ((size_t)b * Hv + h) * kD * kD + (size_t)row * kD + 8 * lq;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                *reinterpret_cast<float4*>(p + 32 * cc) = s0raw[g][cc][0];
                *reinterpret_cast<float4*>(p + 32 * cc + 4) = s0raw[g][cc][1];
            }
        }
    };

    int item = blockIdx.x;                                    // grid <= nitems
    load_small(item, true);
    if constexpr (FUSED) {
        commit_small(item);
        commit_take_small();
        commit_row(item);
    }
    kq_dma(item, true);
#pragma unroll
    for (int g = 0; g < CG; ++g) load_s0(item, g, true);

    for (; item < nitems; item += gridDim.x) {
        asm volatile("" : "+v"(tid));
        lane = tid & 63;
        ln = lane & 15;
        lq = lane >> 4;
        const int nxt = item + gridDim.x;
        const bool more = nxt < nitems;
        const int pf = more ? nxt : item;                     // (the last item: placeholders)
        int b, hk, hg;
        decode(item, b, hk, hg);
        const int h0 = hk * G + hg * HPW;
        const int h = h0 + hp;
        const SeqRows rw = tree_rows(a.offsets, b);
        tn = max(rw.n, 0);
        tbad = rw.n < 0;
        if constexpr (FUSED) prv = tree_rows(c.offsets, b);
        const int tblk = (tn + 15) / 16;                      // this tree's node blocks
        const size_t vo_base = (rw.row0 * Hv + h) * kD;       // node 0 of head h
        lds_barrier();                                        // LDS of the last item is free
        if constexpr (FUSED) {                                // the previous tree's path rows
            commit_path();
            commit_issue(b, hk, h0, 0);
        }

        // ---- 1. tree and path log-gates (wave 0), beta (threads 64 ..) -------
        if (wave == 0) {
            tree_wave();
        } else if (tid < 64 + NP) {
            const int i = tid - 64;
#pragma unroll
            for (int p = 0; p < HPW; ++p)
                s_beta[p][i] = i < tn ? __uint_as_float(sm[NPL + p]) : 0.f;
        }
        // S0 rows (registers) and the direct-to-LDS k / q rows were issued before
        // anything still in flight: one wait covers both, the barrier publishes
        // every wave's copies and the tree.
        wait_vmem_all();
        if constexpr (FUSED) commit_stage(0);
        lds_barrier();
        const int status = __builtin_amdgcn_readfirstlane(s_flag);   // uniform branch below
        if constexpr (FUSED) commit_apply(b, hk, hg, h0, h);
        uint16_t* O = static_cast<uint16_t*>(a.o);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        u32x4 vfr[NB];                                // node 16t + l%16, columns col0 + 8(l/16)..+7
        // this item's S0 rows as bf16 B / A operands (registers for the whole item)
        // (pinned here by an empty asm: sunk to its uses in the solve, the
        // conversion would keep s0raw alive under the next item's prefetch)
        bf16x8 sb[CG][4];
#pragma unroll
        for (int g = 0; g < CG; ++g)
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
                sb[g][cs] = to_bf16x8(s0raw[g][cs][0], s0raw[g][cs][1]);
                asm volatile("" : "+v"(sb[g][cs]));
            }
        const bool solve = status == 0 && tn > 0;          // (an empty tree: nothing to do)
        if (!solve) {
            if (status) {                             // invalid tree: NaN outputs, no solve
                const float qnan = __uint_as_float(0x7fc00000u);
#pragma unroll
                for (int p = 0; p < HPW; ++p) {
                    const size_t ob = (rw.row0 * Hv + h0 + p) * kD;
                    float* Up = a.u + ((size_t)b * Hv + h0 + p) * (size_t)N * kD;
                    for (int x = tid; x < N * kD; x += NT) {
                        if (x < tn * kD) O[ob + (size_t)(x / kD) * vo_row + x % kD] = 0x7fc0;
                        Up[x] = qnan;
                    }
                    for (int i = tid; i < N; i += NT) a.log_gamma[((size_t)b * Hv + h0 + p) * N + i] = qnan;
                }
            }
        } else {
            // this item's v rows, needed only in the solve (unconditional: rows
            // past n re-read row n - 1, and beta = 0 there)
            const uint16_t* V = static_cast<const uint16_t*>(a.v);
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                const int i = min(16 * t + ln, tn - 1);
                vfr[t] = *reinterpret_cast<const u32x4*>(V + vo_base + (size_t)i * vo_row + col0 + 8 * lq);
            }
            // ---- 3. Gram tiles -> masked, decayed X / Y tiles per head ----------
            // Computed transposed, K_s K_t^T and K_s Q_t^T: lane l then holds row
            // i = 16t + l%16 and columns j = 16s + 4(l/16)..+3, which is its place
            // in the tile layout (8 contiguous bytes per lane).  Each wave takes a
            // contiguous run of the (t, s), s <= t, pairs in row order: it keeps row
            // t's k / q fragments across its pairs of that row, and the next pair's
            // fragments are requested before the current pair's masking.
            {
                constexpr int MAXC = (NPAIR + NW - 1) / NW;
                const int p0 = wave * NPAIR / NW, p1 = (wave + 1) * NPAIR / NW;
                int t = 0;
                while ((t + 1) * (t + 2) / 2 <= p0) ++t;
                int s = p0 - t * (t + 1) / 2;
                bf16x8 fk[4], fq[4], fs[4];
#pragma unroll
                for (int cs = 0; cs < 4; ++cs) {
                    fk[cs] = lds_frag(s_k, t, cs, lane);
                    fq[cs] = lds_frag(s_q, t, cs, lane);
                    fs[cs] = lds_frag(s_k, s, cs, lane);
                }
#pragma unroll
                for (int c = 0; c < MAXC; ++c) {
                    if (p0 + c >= p1 || t >= tblk) break;      // uniform
                    f32x4 A = z, C = z;
#pragma unroll
                    for (int cs = 0; cs < 4; ++cs) {
                        A = mfma32(fs[cs], fk[cs], A);
                        C = mfma32(fs[cs], fq[cs], C);
                    }
                    const int tc = t, sc = s;
                    // the next pair's fragments (rows past N re-read earlier
                    // rows: harmless, never used)
                    if (++s > t) { ++t; s = 0; }
                    if (c + 1 < MAXC) {
                        const int tl = min(t, NB - 1);
                        if (s == 0) {
#pragma unroll
                            for (int cs = 0; cs < 4; ++cs) {
                                fk[cs] = lds_frag(s_k, tl, cs, lane);
                                fq[cs] = lds_frag(s_q, tl, cs, lane);
                            }
                        }
#pragma unroll
                        for (int cs = 0; cs < 4; ++cs) fs[cs] = lds_frag(s_k, min(s, NB - 1), cs, lane);
                    }
                    const int i = 16 * tc + ln, j0 = 16 * sc + 4 * lq;
                    const uint32_t bits = i < tn ? (s_mask[i * MW + (j0 >> 5)] >> (j0 & 31)) & 15u : 0u;
#pragma unroll
                    for (int p = 0; p < HPW; ++p) {
                        const float lgi = s_lg[p][i], bei = s_beta[p][i];
                        const float4 lgj = *reinterpret_cast<const float4*>(&s_lg[p][j0]);
                        const float lj[4] = {lgj.x, lgj.y, lgj.z, lgj.w};
                        float xv[4];
                        uint16_t yv[4], nxv[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const bool anc = (bits >> e) & 1u;
                            const bool self = (j0 + e == i) && i < tn;
                            const float d = (anc || self) ? __expf(lgi - lj[e]) : 0.f;
                            xv[e] = anc ? bei * d * A[e] : 0.f;
                            yv[e] = bf16_rne(d * C[e]);
                            nxv[e] = bf16_rne(-xv[e]);
                        }
                        const int tp = a32_pos(ln, 4 * lq);       // 4 consecutive columns: 8 bytes
                        *reinterpret_cast<uint2*>(&s_tiles[p][(NX + tc * (tc + 1) / 2 + sc) * 256 + tp]) =
                            make_uint2(yv[0] | ((uint32_t)yv[1] << 16), yv[2] | ((uint32_t)yv[3] << 16));
                        if (sc < tc)
                            *reinterpret_cast<uint2*>(&s_tiles[p][(tc * (tc - 1) / 2 + sc) * 256 + tp]) =
                                make_uint2(nxv[0] | ((uint32_t)nxv[1] << 16), nxv[2] | ((uint32_t)nxv[3] << 16));
                        else
                            *reinterpret_cast<float4*>(&s_xd[p][tc * 256 + ln * 16 + 4 * lq]) =
                                make_float4(xv[0], xv[1], xv[2], xv[3]);
                    }
                }
            }
            lds_barrier();

        }
        // s0raw is free: the next item's parent / g / beta and S0 rows load
        // during the inversion, ahead of the solve's output stores (loads and
        // stores retire in order).  One program point for both paths, so no
        // register copy of a load in flight is needed where they meet.
        load_small(pf, more);
        if constexpr (FUSED) {
            commit_small(pf);
            // (fused: the next item's S0 rows right here; spread over the solve
            // they would meet the committed rows' stores less well)
#pragma unroll
            for (int g = 0; g < CG; ++g) load_s0(pf, g, more);
        }
        if (solve) {
            // ---- 4. diagonal blocks: (I + X_tt)^-1 in fp32 ----------------------
            for (int blk = tid >> 4; blk < HPW * NB; blk += NT / 16) {
                const int p = blk / NB, t = blk % NB;
                if (t < tblk) {
                    const float* xd = s_xd[p] + t * 256;
                    float y[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float acc = (i == ln) ? 1.f : 0.f;
#pragma unroll
                        for (int m = 0; m < i; ++m) acc = fmaf(-xd[i * 16 + m], y[m], acc);
                        y[i] = acc;
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) s_dinv[p][t * 256 + a32_pos(i, ln)] = bf16_rne(y[i]);
                }
            }
            lds_barrier();
        }
        // v landed: only the next item's small loads (and, fused, its S0 rows),
        // issued after it, may still be in flight (the explicit count lets them
        // overlap the solve).
        wait_vmem_le<FUSED ? NSM + 2 + 8 * CG : NSM>();
        if constexpr (FUSED) commit_take_small();
        if (wave == NW - 1) write_tree_cache(b, h0, hk == 0 && hg == 0, status);
        // ---- 5. per wave: projection, blocked substitution, output ---------
        //   sb[g][cs]   S0 rows of group g (local row l%16): B operand of K S0^T, A
        //               operand of S0 Q^T;  k / q frags of block t (LDS): A / B;
        //   vfr[t]      v rows of block t, both groups' columns; group g's half
        //               (A operand) is moved into accumulator layout by an exact
        //               product with I;
        //   up[g][p]    [U_2p; U_2p+1] rounded to bf16 as a 16x16x32 B operand
        //               (stack_pair): B operand of [X_t,2p | X_t,2p+1] U and,
        //               read as [U_2p^T | U_2p+1^T], A operand of U^T Y^T.  Until
        //               U_2p+1 exists its half is zero.  U itself (stored to the
        //               cache) stays fp32: R_t is split into bf16 hi + lo and
        //               [D | D] [hi; lo] is one MFMA, D = (I + X_tt)^-1.
        //   Every tile product takes two node blocks at once (K = 32); a row's
        //   last pair with one block only has its second half zeroed.
        const uint16_t* tiles = s_tiles[hp];
        const float* lgp = s_lg[hp];
        const float* bep = s_beta[hp];
        float* Ug = a.u + ((size_t)b * Hv + h) * (size_t)N * kD;
        const s16x4 zero4 = {0, 0, 0, 0};
        const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        const bool hi_half = lq >= 2;                          // lanes of the pair's second block
        bf16x8 up[CG][(NB + 1) / 2];
        const int nsolve = solve ? tblk : 0;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            // (not fused) the next item's S0 rows, one column group at a time,
            // spread over the solve so that their reads share the HBM with its
            // stores
            if constexpr (!FUSED) {
                if (t == NB / 4) load_s0(pf, 0, more);
                if (t == NB / 2) load_s0(pf, 1, more);
            }
            if (t >= nsolve) continue;                        // uniform
            f32x4 pk[CG], pqT[CG];
#pragma unroll
            for (int g = 0; g < CG; ++g) pk[g] = pqT[g] = z;
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
                const bf16x8 kf = lds_frag(s_k, t, cs, lane), qf = lds_frag(s_q, t, cs, lane);
#pragma unroll
                for (int g = 0; g < CG; ++g) {
                    pk[g] = mfma32(kf, sb[g][cs], pk[g]);           // [node][r]
                    pqT[g] = mfma32(sb[g][cs], qf, pqT[g]);         // [r][node]
                }
            }
            f32x4 R[CG];
#pragma unroll
            for (int g = 0; g < CG; ++g) {
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 vg = {vfr[t][2 * g], vfr[t][2 * g + 1]};   // group g's 4 columns
                const f32x4 vd = mfma16(__builtin_bit_cast(s16x4, vg), ident, z);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int i = 16 * t + 4 * lq + m;
                    R[g][m] = bep[i] * (vd[m] - __expf(lgp[i]) * pk[g][m]);
                }
            }
            // R_t += sum_{s<t} (-X_ts) U_s, two blocks per product
#pragma unroll
            for (int s = 0; s < t; s += 2) {
                bf16x8 nx = *reinterpret_cast<const bf16x8*>(tiles + (t * (t - 1) / 2 + s) * 256 + lane * 8);
                if (s + 1 == t) nx = hi_half ? zero8 : nx;        // X_tt is not in the sum
#pragma unroll
                for (int g = 0; g < CG; ++g) R[g] = mfma32(nx, up[g][s / 2], R[g]);
            }
            // U_t = D R_t, kept as [node][r]; U_t^T = R_t^T D^T is stored
            const bf16x8 di = *reinterpret_cast<const bf16x8*>(s_dinv[hp] + t * 256 + (ln + 16 * (lq & 1)) * 8);
            const int node = 16 * t + ln;                     // this lane's node in ^T tiles
#pragma unroll
            for (int g = 0; g < CG; ++g) {
                s16x4 rh, rl;
                split4(R[g], rh, rl);
                const bf16x8 rr = stack_pair(rh, rl);
                const f32x4 U = mfma32(di, rr, z);
                const f32x4 UT = mfma32(rr, di, z);
                // (the halves of a stacked pair sit in disjoint lanes: the odd
                // block is OR-ed into the pair its even partner started)
                const s16x4 ut = to_bf16x4(U);
                if (t & 1)
                    up[g][t / 2] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, up[g][t / 2]) |
                                                                  __builtin_bit_cast(u32x4, stack_pair(zero4, ut)));
                else
                    up[g][t / 2] = stack_pair(ut, zero4);
                if (node < tn) *reinterpret_cast<f32x4*>(Ug + (size_t)node * kD + col0 + 8 * lq + 4 * g) = UT;
            }
            // O_t^T = e^G P_Q^T + sum_{s<=t} U_s^T Y_ts^T, two blocks per product
            f32x4 Oc[CG];
#pragma unroll
            for (int g = 0; g < CG; ++g) Oc[g] = z;
#pragma unroll
            for (int s = 0; s <= t; s += 2) {
                bf16x8 yt = *reinterpret_cast<const bf16x8*>(tiles + (NX + t * (t + 1) / 2 + s) * 256 + lane * 8);
                if (s == t) yt = hi_half ? zero8 : yt;            // no block t + 1 in row t
#pragma unroll
                for (int g = 0; g < CG; ++g) Oc[g] = mfma32(up[g][s / 2], yt, Oc[g]);
            }
            if (node < tn) {
                const float egn = __expf(lgp[node]);
                u32x4 ov;
#pragma unroll
                for (int g = 0; g < CG; ++g) {
                    f32x4 OT;
#pragma unroll
                    for (int m = 0; m < 4; ++m) OT[m] = egn * pqT[g][m] + Oc[g][m];
                    ov[2 * g] = (uint32_t)bf16_rne(OT[0]) | ((uint32_t)bf16_rne(OT[1]) << 16);
                    ov[2 * g + 1] = (uint32_t)bf16_rne(OT[2]) | ((uint32_t)bf16_rne(OT[3]) << 16);
                }
                *reinterpret_cast<u32x4*>(O + vo_base + (size_t)node * vo_row + col0 + 8 * lq) = ov;
            }
        }
        lds_barrier();                                      // k / q in LDS are free now
        if constexpr (FUSED) commit_row(pf);                  // ahead of the k / q rows
        // the next item's k / q.  Fused: issued after the last item too, so that
        // every path into the next item has the same loads in flight after the
        // ancestor row (the wait for it then leaves the copies running)
        if constexpr (FUSED) kq_dma(pf, more);
        else if (more) kq_dma(nxt, true);
    }
}

}  // namespace

bool verify_tiled_supported(const VerifyArgs& a, int io) {
    return io == GDN_BF16 && a.dk == kD && a.dv == kD && a.N <= 128;
}

template <bool FUSED, bool RAGGED>
static const void* tiled_kernel(int N, int hpw) {
    if (N <= 64)
        return hpw == 2 ? (const void*)verify_tiled_kernel<4, 2, FUSED, RAGGED>
                        : (const void*)verify_tiled_kernel<4, 1, FUSED, RAGGED>;
    return hpw == 2 ? (const void*)verify_tiled_kernel<8, 2, FUSED, RAGGED>
                    : (const void*)verify_tiled_kernel<8, 1, FUSED, RAGGED>;
}

template <bool FUSED>
static hipError_t launch_tiled(const VerifyArgs& a, const CommitArgs& c, hipStream_t stream) {
    const int G = a.Hv / a.Hk;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // Two value heads per workgroup where G allows it, except for trees of up
    // to 64 nodes when that would leave compute units idle: there one head per
    // workgroup, two workgroups per compute unit (49 KB of LDS and at most 256
    // registers per lane each), spreads a small batch over twice the units.
    const bool small = a.N <= 64 && a.B * a.Hk * (G / 2) < cus;
    const int hpw = (G % 2 == 0 && !small) ? 2 : 1;
    // ragged: the new tree's offsets, and (fused) the previous tree's as well
    const bool ragged = a.offsets != nullptr;
    if (FUSED && ragged != (c.offsets != nullptr)) return hipErrorInvalidValue;
    const void* fn = ragged ? tiled_kernel<FUSED, true>(a.N, hpw) : tiled_kernel<FUSED, false>(a.N, hpw);
    int nitems = a.B * a.Hk * (G / hpw);
    const int slots = (a.N <= 64 && hpw == 1) ? 2 * cus : cus;
    const unsigned grid = (unsigned)(nitems < slots ? nitems : slots);
    VerifyArgs va = a;
    CommitArgs ca = c;
    void* args[] = {&va, &ca, &nitems};
    return hipLaunchKernel(fn, dim3(grid), dim3(256 * hpw), args, 0, stream);
}

hipError_t launch_verify_tiled(const VerifyArgs& a, int io, hipStream_t stream) {
    (void)io;
    return launch_tiled<false>(a, CommitArgs{}, stream);
}

hipError_t launch_commit_verify_tiled(const VerifyArgs& a, const CommitArgs& c, int io, hipStream_t stream) {
    (void)io;
    return launch_tiled<true>(a, c, stream);
}

}  // namespace gdn
