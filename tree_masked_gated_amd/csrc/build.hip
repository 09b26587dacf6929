// build.hip -- draft-tree construction with w expansions per step, on the
// device (page "Trees from Marginals: Autoregressive drafting with factorized
// priors", section 2, tree construction: DySpec's best-first expansion, changed
// so that the w best candidates leave the candidate heap together and are
// expanded together; a tree of N nodes takes ceil(N / w) sequential steps).
// The drafter's outputs are inputs here: for the prefix (row 0) and for every
// node index i (row 1 + i), its K continuations as log-probabilities and
// tokens.  A candidate is the continuation of rank c after a placed node p
// (p = -1: the prefix), scored score(p) + logp[p + 1][c] in fp32 with
// score(prefix) = 0; a step takes the min(w, nodes left, candidates) best,
// ordered by score, then parent, then rank, as nodes n, n + 1, ...
//
// One workgroup of eight waves per sequence: a step's work is spread over
// all its threads, so a step costs about one binary search per thread.  The
// sequence's log-probability table is staged in LDS once.  A candidate is one
// 64-bit key whose unsigned order is the selection order (order-preserving
// score bits, then 0xffff - (p + 1), then 0xffff - c); keys are distinct, so
// no tie needs a rule of its own.  The open candidates are one list sorted in
// descending key order.  A step's new children are sorted by rank (a key's
// place is the number of larger keys) and merged into the list by rank (a
// key's place is its index in its own list plus the number of larger keys in
// the other, a binary search, one key per thread), and the list is cut to
// the nodes still to place: a candidate with that many better ones can never
// be chosen.  Steps of up to 64 children overlap: the step's new nodes are
// the best of the two lists' heads, so two waves rank the next step's
// children while the others merge (one barrier per step).
#include "gdn_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int kBuildThreads = 512;

// order-preserving 32-bit image of a finite (or infinite) float; -0 counts as +0
__device__ __forceinline__ uint32_t score_bits(float s) {
    const uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffffu) == 0u) return 0x80000000u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float bits_score(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ uint64_t cand_key(float s, int p, int c) {
    return ((uint64_t)score_bits(s) << 32) | ((uint64_t)(0xffffu - (uint32_t)(p + 1)) << 16) |
           (uint64_t)(0xffffu - (uint32_t)c);
}
__device__ __forceinline__ int key_parent(uint64_t k) { return (int)(0xffffu - ((uint32_t)(k >> 16) & 0xffffu)) - 1; }
__device__ __forceinline__ int key_rank(uint64_t k) { return (int)(0xffffu - ((uint32_t)k & 0xffffu)); }

// number of keys of x[0 .. n) (descending, distinct) larger than key
__device__ __forceinline__ int count_larger(const uint64_t* x, int n, uint64_t key) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (x[mid] > key) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Number of lanes Y0 <= y < Y0 + CNT of the calling wave whose key is
// larger than this lane's (every other lane's key read into scalar
// registers; no LDS).  Lanes without a key hold 0, below every key.
template <int CNT, int Y0 = 0>
__device__ __forceinline__ int lanes_larger(uint64_t key) {
    const uint32_t klo = (uint32_t)key, khi = (uint32_t)(key >> 32);
    int r = 0;
#pragma unroll
    for (int y = Y0; y < Y0 + CNT; ++y) {
        const uint64_t ky = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)khi, y) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)klo, y);
        r += ky > key ? 1 : 0;
    }
    return r;
}

struct BuildLds {
    int N, K, P;              // nodes, continuations per row, child keys per step
    __host__ __device__ BuildLds(int n, int k, int p) : N(n), K(k), P(p) {}
    // byte offsets: two lists of N keys, P child keys twice (as formed, then
    // sorted), then the table and per-node words
    __host__ __device__ size_t list(int i) const { return (size_t)i * N * 8; }
    __host__ __device__ size_t child(int i) const { return list(2) + (size_t)i * P * 8; }
    __host__ __device__ size_t table() const { return child(2); }
    __host__ __device__ size_t score() const { return table() + (size_t)(N + 1) * K * 4; }
    __host__ __device__ size_t parent() const { return score() + (size_t)N * 4; }
    __host__ __device__ size_t rank() const { return parent() + (size_t)N * 4; }
    // a step's new nodes (two copies of 32 keys), then 64 partial ranks and a flag
    __host__ __device__ size_t top() const { return rank() + (size_t)N * 4; }
    __host__ __device__ size_t part() const { return top() + 2 * 32 * 8; }
    __host__ __device__ size_t bytes() const { return part() + 65 * 4; }
};

__global__ __launch_bounds__(kBuildThreads) void tree_build_kernel(BuildArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int N = a.N, K = a.K, w = a.w;
    const int wn = w < N ? w : N;
    const BuildLds L(N, K, wn * K);
    // (the lists are addressed from one LDS base: a pointer picked from an
    // array would lose its address space and turn every access into a flat one)
    uint64_t* lists = reinterpret_cast<uint64_t*>(smem + L.list(0));    // [2][N]
    uint64_t* cu = reinterpret_cast<uint64_t*>(smem + L.child(0));    // this step's children
    uint64_t* ck = reinterpret_cast<uint64_t*>(smem + L.child(1));    // the same, sorted
    float* lp = reinterpret_cast<float*>(smem + L.table());
    float* sc = reinterpret_cast<float*>(smem + L.score());
    int32_t* par = reinterpret_cast<int32_t*>(smem + L.parent());
    int32_t* rk = reinterpret_cast<int32_t*>(smem + L.rank());
    const int b = blockIdx.x, tid = threadIdx.x;
    const size_t rows = (size_t)(N + 1) * K;

    const float* g_lp = a.logp + (size_t)b * rows;
    for (size_t x = tid; x < rows; x += kBuildThreads) lp[x] = g_lp[x];
    for (int i = tid; i < N; i += kBuildThreads) {
        par[i] = -1;
        rk[i] = 0;
        sc[i] = 0.0f;
    }
    __syncthreads();

    int cur = 0, head = 0, len = 0;        // open candidates: lists[cur N + head .. cur N + len)
    int n = 0, e0 = -1, ne = 1;            // the nodes to expand: e0 .. e0 + ne - 1 (-1: the prefix)
    if (L.P <= 64 && wn <= 32) {
        // Steps of up to 64 children, pipelined: once a step's children are
        // sorted, its new nodes are the best m of the heads of the two sorted
        // lists (the first m open candidates and the first m children), so
        // wave 0 finds them and sorts the next step's children while the
        // other waves merge the whole lists.  One barrier per step.
        uint64_t* cks = reinterpret_cast<uint64_t*>(smem + L.child(0));   // [2][P] sorted children
        uint64_t* top = reinterpret_cast<uint64_t*>(smem + L.top());       // [2][32] a step's new nodes
        int* part = reinterpret_cast<int*>(smem + L.part());               // [64] counts, [64] flag
        int cb = 0;                        // this step's children: cks[cb P ..]
        int nstep = 0;                     // this step's number, from 1 (the flag's value)
        if (tid == 0) part[64] = 0;
        if (tid < 64) {                    // the prefix's children
            const uint64_t key = tid < K ? cand_key(0.0f + lp[tid], -1, tid) : 0;
            const int r = lanes_larger<64>(key);
            if (tid < K) cks[r] = key;
        }
        __syncthreads();
        for (;;) {
            ++nstep;
            const int nc = ne * K;
            const uint64_t* ck = cks + (size_t)cb * L.P;
            const int R = N - n;
            const uint64_t* A = lists + (size_t)cur * N + head;
            const int na = len - head;
            uint64_t* out = lists + (size_t)(cur ^ 1) * N;
            len = min(na + nc, R);
            const int m = min(min(w, R), len);
            if (tid < 128) {
                // waves 0 and 1 both: this step's new nodes, lanes 0 .. m-1
                // holding the first m open candidates and lanes m .. 2m-1 the
                // first m children (0 past either list: below every key);
                // then their children, the next step's, ranked by wave 0 over
                // lanes 0 .. 31 and wave 1 over lanes 32 .. 63, wave 1's
                // counts handed over through LDS under a step-numbered flag
                if (n + m < N) {
                    const int ln = tid & 63, wv = tid >> 6;
                    uint64_t key = 0;
                    if (ln < m) key = ln < na ? A[ln] : 0;
                    else if (ln < 2 * m) key = ln - m < nc ? ck[ln - m] : 0;
                    const int r = 2 * m <= 16 ? lanes_larger<16>(key)
                                  : 2 * m <= 32 ? lanes_larger<32>(key) : lanes_larger<64>(key);
                    uint64_t* topw = top + 32 * wv;
                    if (key != 0 && r < m) topw[r] = key;
                    const int nc2 = m * K;
                    uint64_t k2 = 0;
                    if (ln < nc2) {
                        const int t = ln / K, c = ln - t * K;
                        const uint64_t kt = topw[t];
                        const int pn = n + t;
                        k2 = cand_key(bits_score((uint32_t)(kt >> 32)) + lp[(size_t)(pn + 1) * K + c], pn, c);
                    }
                    if (wv == 1) {
                        part[ln] = lanes_larger<32, 32>(k2);
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                        if (ln == 0) __hip_atomic_store(&part[64], nstep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    } else {
                        const int r0 = lanes_larger<32>(k2);
                        while (__hip_atomic_load(&part[64], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != nstep)
                            __builtin_amdgcn_s_sleep(1);
                        asm volatile("" ::: "memory");
                        if (ln < nc2) cks[(size_t)(cb ^ 1) * L.P + r0 + part[ln]] = k2;
                    }
                }
            } else {
                // the merge by rank (a key's place: its index in its own list
                // plus the number of larger keys in the other, a binary
                // search), keeping the best N - n; the thread placing one of
                // the best m records it as node n + pos
                for (int x = tid - 128; x < na + nc; x += kBuildThreads - 128) {
                    const bool open = x < na;
                    const uint64_t key = open ? A[x] : ck[x - na];
                    const int pos = open ? x + count_larger(ck, nc, key) : x - na + count_larger(A, na, key);
                    if (pos < R) out[pos] = key;
                    if (pos < m) {
                        sc[n + pos] = bits_score((uint32_t)(key >> 32));
                        par[n + pos] = key_parent(key);
                        rk[n + pos] = key_rank(key);
                    }
                }
            }
            __syncthreads();
            if (m == 0 || n + m >= N) break;   // (m = 0 never: every step adds K >= 1 candidates)
            cur ^= 1;
            cb ^= 1;
            e0 = n;
            ne = m;
            head = m;
            n += m;
        }
    } else {
        for (;;) {
            // 1. the expanded nodes' children, as keys, sorted descending: each
            // key's place is the number of larger ones.  Up to 64 children: one
            // wave, key x in lane x, every other lane's key taken by a lane read
            // into scalar registers (no LDS round trip); more: a scan of the keys
            // in LDS, every lane of a wave reading the same key at once.
            const int nc = ne * K;
            auto child_key = [&](int x) {
                const int t = x / K, c = x - t * K;
                const int p = e0 < 0 ? -1 : e0 + t;
                const float base = p < 0 ? 0.0f : sc[p];
                return cand_key(base + lp[(size_t)(p + 1) * K + c], p, c);
            };
            if (nc <= 64) {
                if (tid < 64) {
                    const uint64_t key = tid < nc ? child_key(tid) : 0;
                    const uint32_t klo = (uint32_t)key, khi = (uint32_t)(key >> 32);
                    int r = 0;
    #pragma unroll
                    for (int y = 0; y < 64; ++y) {
                        const uint64_t ky = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)khi, y) << 32) |
                                            (uint32_t)__builtin_amdgcn_readlane((int)klo, y);
                        r += ky > key ? 1 : 0;     // (lanes past nc hold 0: never larger)
                    }
                    if (tid < nc) ck[r] = key;
                }
            } else {
                for (int x = tid; x < nc; x += kBuildThreads) cu[x] = child_key(x);
                __syncthreads();
                for (int x = tid; x < nc; x += kBuildThreads) {
                    const uint64_t key = cu[x];
                    int r = 0;
    #pragma unroll 8
                    for (int y = 0; y < nc; ++y) r += cu[y] > key ? 1 : 0;
                    ck[r] = key;
                }
            }
            __syncthreads();
            // 2. merge into the open list, keeping the best N - n (a key's place:
            // its index in its own list plus the number of larger keys in the
            // other, a binary search; one key per thread); 3. the step: the best
            // m open candidates become nodes n .. n + m - 1, recorded by
            // whichever thread places them
            const int R = N - n;
            const uint64_t* A = lists + (size_t)cur * N + head;
            const int na = len - head;
            uint64_t* out = lists + (size_t)(cur ^ 1) * N;
            len = min(na + nc, R);
            const int m = min(min(w, R), len);
            for (int x = tid; x < na + nc; x += kBuildThreads) {
                const bool open = x < na;
                const uint64_t key = open ? A[x] : ck[x - na];
                const int pos = open ? x + count_larger(ck, nc, key) : x - na + count_larger(A, na, key);
                if (pos < R) out[pos] = key;
                if (pos < m) {
                    sc[n + pos] = bits_score((uint32_t)(key >> 32));
                    par[n + pos] = key_parent(key);
                    rk[n + pos] = key_rank(key);
                }
            }
            cur ^= 1;
            head = 0;
            __syncthreads();
            if (m == 0) break;                 // (never: every step adds K >= 1 candidates)
            e0 = n;
            ne = m;
            head = m;
            n += m;
            if (n >= N) break;
        }
    }
    // the tree, with each node's token from its parent's row
    const int32_t* g_tok = a.tok + (size_t)b * rows;
    for (int i = tid; i < N; i += kBuildThreads) {
        const int p = par[i];
        a.parent[(size_t)b * N + i] = p;
        a.token[(size_t)b * N + i] = g_tok[(size_t)(p + 1) * K + rk[i]];
        a.score[(size_t)b * N + i] = sc[i];
    }
}

}  // namespace

size_t tree_build_lds_bytes(int N, int K, int w) {
    const int wn = w < N ? w : N;
    return BuildLds(N, K, wn * K).bytes();
}

hipError_t launch_tree_build(const BuildArgs& a, hipStream_t stream) {
    const size_t lds = tree_build_lds_bytes(a.N, a.K, a.w);
    if (lds > (size_t)kMaxLds) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void*)tree_build_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    BuildArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel((const void*)tree_build_kernel, dim3((unsigned)a.B), dim3(kBuildThreads),
                           args, lds, stream);
}

}  // namespace gdn
