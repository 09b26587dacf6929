// gdn_common.hpp -- device helpers shared by the gfx950 kernels of the GDN
// draft-tree library: element codecs, kernel argument blocks and the
// in-LDS construction of a tree's ancestor bit rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_tree.h"

namespace gdn {

constexpr int kMaxNodes = 1024;     // largest tree one call accepts
constexpr int kMaxHead = 256;       // largest d_k / d_v one call accepts
constexpr int kMaxLds = 160 * 1024; // LDS bytes a gfx950 workgroup may hold

struct VerifyArgs {
    int B, N, Hk, Hv, dk, dv;
    const float* S0;
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    const float* g;
    const int32_t* parent;
    void* o;
    uint32_t* anc_mask;
    int32_t* depth;
    float* u;
    float* log_gamma;
    int32_t* status;
    const int32_t* offsets;   // ragged layout: [B + 1] first rows; nullptr = dense
};

struct CommitArgs {
    int B, N, Hk, Hv, dk, dv;
    const float* S_in;
    float* S_out;
    const void* k;
    const uint32_t* anc_mask;
    const float* u;
    const float* log_gamma;
    const int32_t* status;
    const int32_t* accepted;
    int32_t* path;
    int32_t* path_len;
    const int32_t* offsets;   // ragged layout of k and path; nullptr = dense
};

// Rows of sequence b in the per-node arrays (q, k, v, o, beta, g, parent, the
// acceptance tokens and a commit's path).  Dense layout (offsets = nullptr):
// rows b N .. b N + N - 1.  Ragged layout: rows offsets[b] .. offsets[b+1] - 1,
// N being the largest tree; n = -1 marks a sequence whose offsets are unusable
// (a negative first row, or a node count outside [0, N]), and then nothing of
// it is read.  b must be uniform over the wave: the two offsets are read
// through the scalar cache, so waiting for them does not wait for the wave's
// vector loads.
struct SeqRows {
    int64_t row0;
    int n;
};
__device__ __forceinline__ SeqRows seq_rows(const int32_t* offsets, int b, int N) {
    if (offsets == nullptr) return SeqRows{(int64_t)b * N, N};
    typedef __attribute__((address_space(4))) const int32_t cint32;
    const cint32* p = (const cint32*)offsets;
    const int64_t o0 = p[b], n = (int64_t)p[b + 1] - o0;
    if (o0 < 0 || n < 0 || n > N) return SeqRows{0, -1};
    return SeqRows{o0, (int)n};
}

// ------------------------------------------------------------- element codecs

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t x = __float_as_uint(f);
    if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
    x += 0x7fffu + ((x >> 16) & 1u);
    return (uint16_t)(x >> 16);
}

// IO = GDN_F32 or GDN_BF16: element i of a q/k/v/o array as fp32.
template <int IO>
__device__ __forceinline__ float ld_io(const void* p, size_t i) {
    if constexpr (IO == GDN_BF16)
        return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    else
        return static_cast<const float*>(p)[i];
}

template <int IO>
__device__ __forceinline__ void st_io(void* p, size_t i, float x) {
    if constexpr (IO == GDN_BF16)
        static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x);
    else
        static_cast<float*>(p)[i] = x;
}

// ------------------------------------------------------------- tree in LDS

__device__ __forceinline__ int lds_load_acquire(int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store_release(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint32_t lds_load_relaxed(uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store_relaxed(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Workgroup barrier that orders LDS only: this wave's LDS operations are
// complete, then all waves meet.  Unlike __syncthreads() it does not wait for
// the wave's outstanding global loads and stores, so prefetches and output
// stores stay in flight across it.  Only valid where no thread reads global
// memory written by another thread of the workgroup.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until every global load and store of this wave has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima).  Issued through
// the builtin rather than inline asm so that the compiler's own wait
// insertion knows the loads are done, in particular the direct-to-LDS loads,
// which it otherwise waits for again before later LDS reads.
__device__ __forceinline__ void wait_vmem_all() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Wait until at most n global loads / stores of this wave are in flight
// (they retire in issue order): a compile-time n, encoded for gfx9 s_waitcnt.
template <int n>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// Validate one tree's parent row and build its strict-ancestor bit rows in LDS
// (the ancestor relation behind the interaction matrices X and Y).
//
// mask: N * W words (W = ceil(N/32)), jump: N ints, s_flag: one int, all LDS.
// Returns the tree status (0 valid, else i + 1 for the first node i whose
// parent lies outside [-1, i)), the same value in every thread.  Rows are
// left zero for an invalid tree.
//
// Rows are filled by pointer jumping done in place: the owner of row i keeps
// a pointer J_i to an ancestor such that row i already holds every node on the
// path from parent(i) up to and including J_i; one step ORs in row J_i and
// moves J_i to J_(J_i).  Row words are published before the pointer (release /
// acquire), so a reader that sees a pointer also sees the words it covers;
// seeing a later value of either only adds true ancestors.  Every step moves
// J_i strictly rootward, so the loop ends; the segment at least doubles per
// round, so ceil(log2(N)) + 1 rounds suffice.
// kLdsOnly selects lds_barrier() (parent row already in LDS, nothing global
// read here) instead of __syncthreads().
template <bool kLdsOnly = false>
__device__ inline int tree_build_lds(const int32_t* __restrict__ par, int N, int W,
                                     uint32_t* mask, int32_t* jump, int* s_flag) {
    auto bar = [] {
        if constexpr (kLdsOnly) lds_barrier(); else __syncthreads();
    };
    const int tid = threadIdx.x, nt = blockDim.x;
    if (tid == 0) *s_flag = 0x7fffffff;
    for (int x = tid; x < N * W; x += nt) mask[x] = 0u;
    bar();
    for (int i = tid; i < N; i += nt) {
        int p = par[i];
        jump[i] = p;
        if (p < -1 || p >= i) atomicMin(s_flag, i);
    }
    bar();
    const int first_bad = *s_flag;
    bar();
    if (first_bad != 0x7fffffff) return first_bad + 1;

    for (int i = tid; i < N; i += nt) {
        int p = jump[i];
        if (p >= 0) mask[i * W + (p >> 5)] = 1u << (p & 31);
    }
    bar();
    for (int round = 0; round < 12; ++round) {
        int active = 0;
        for (int i = tid; i < N; i += nt) {
            const int j = jump[i];
            if (j < 0) continue;
            const int nxt = lds_load_acquire(&jump[j]);
            for (int w = 0; w < W; ++w) {
                uint32_t mine = mask[i * W + w];
                uint32_t theirs = lds_load_relaxed(&mask[j * W + w]);
                if (theirs & ~mine) lds_store_relaxed(&mask[i * W + w], mine | theirs);
            }
            lds_store_release(&jump[i], nxt);
            active |= (nxt >= 0);
        }
        // any thread still jumping?  (s_flag is free after the validity check)
        if (tid == 0) *s_flag = 0;
        bar();
        if (active) *s_flag = 1;
        bar();
        const int any = *s_flag;
        bar();
        if (!any) break;
    }
    return 0;
}

// Index of the m-th set bit (0-based, ascending) of a W-word row.
__device__ __forceinline__ int nth_set_bit(const uint32_t* row, int W, int m) {
    for (int w = 0; w < W; ++w) {
        uint32_t x = row[w];
        int c = __popc(x);
        if (m < c) {
            for (int t = 0; t < m; ++t) x &= x - 1u;
            return w * 32 + __ffs(x) - 1;
        }
        m -= c;
    }
    return -1;
}

__device__ __forceinline__ int row_popc(const uint32_t* row, int W) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popc(row[w]);
    return c;
}

// In-place inclusive prefix sum of x[0..n) by the whole workgroup; part holds
// blockDim.x ints of LDS scratch.  Ends with a barrier.
__device__ inline void block_inclusive_scan(int32_t* x, int n, int* part) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int seg = (n + nt - 1) / nt;
    const int s = min(n, tid * seg), e = min(n, s + seg);
    int local = 0;
    for (int t = s; t < e; ++t) local += x[t];
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < nt; off <<= 1) {
        int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int run = tid ? part[tid - 1] : 0;
    for (int t = s; t < e; ++t) {
        run += x[t];
        x[t] = run;
    }
    __syncthreads();
}

}  // namespace gdn
