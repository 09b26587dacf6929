// verify_generic.hip -- general-shape tree verification kernel (fp32 vector
// arithmetic) for every size the library accepts: any tree of up to 1024
// nodes, head sizes up to 256, fp32 or bf16 q/k/v/o.
//
// Method (page "Trees from Marginals: Autoregressive drafting with factorized
// priors", section 3, rollback-free tree verification for GDN): the tree's
// ancestor relation gives the interaction matrices
//     X_ij = beta_i e^(G_i - G_j) k_i.k_j   (j a strict ancestor of i)
//     Y_ij = e^(G_i - G_j) q_i.k_j          (j an ancestor of i, or i itself)
// with G_i the path sum of ln g; the masked unit-lower-triangular system
// (I + X) U = R, R = diag(beta)(V - diag(e^G) K S0^T), is solved by forward
// substitution in topological (depth) order, and the outputs are
// O = diag(e^G) Q S0^T + Y U.  Nothing writes S0.
//
// One workgroup per (sequence, value head).  The tree's ancestor rows live in
// LDS; U lives in the caller's cache buffer (global memory, L2-resident while
// the workgroup runs).  Nodes are processed level by level; a level is split
// into chunks whose X (or Y) coefficients fit in LDS.
#include "gdn_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kCoefCap = 512;    // X / Y coefficients staged per chunk

// LDS layout of the generic kernel, in 4-byte words.
struct GenericLds {
    int N, W;
    __device__ __host__ GenericLds(int n) : N(n), W((n + 31) / 32) {}
    __device__ __host__ int mask() const { return 0; }
    __device__ __host__ int jump() const { return N * W; }
    __device__ __host__ int lg() const { return jump() + N; }
    __device__ __host__ int lng() const { return lg() + N; }
    __device__ __host__ int dep() const { return lng() + N; }
    __device__ __host__ int order() const { return dep() + N; }
    __device__ __host__ int lvl() const { return order() + N; }      // N + 1 offsets
    __device__ __host__ int coef() const { return lvl() + N + 1; }
    __device__ __host__ int cidx() const { return coef() + kCoefCap; }
    __device__ __host__ int words() const { return cidx() + kCoefCap; }
};

template <int IO>
__global__ __launch_bounds__(kThreads) void verify_generic_kernel(VerifyArgs a) {
    extern __shared__ uint32_t smem[];
    __shared__ int s_flag;
    __shared__ int s_maxdep;
    __shared__ int s_part[kThreads];
    __shared__ float s_acc[kMaxHead];

    const int N = a.N, dk = a.dk, dv = a.dv;
    const GenericLds L(N);
    const int W = L.W;
    uint32_t* mask = smem + L.mask();
    int32_t* jump = reinterpret_cast<int32_t*>(smem + L.jump());
    float* lg = reinterpret_cast<float*>(smem + L.lg());
    float* lng = reinterpret_cast<float*>(smem + L.lng());
    int32_t* dep = reinterpret_cast<int32_t*>(smem + L.dep());
    int32_t* order = reinterpret_cast<int32_t*>(smem + L.order());
    int32_t* lvl = reinterpret_cast<int32_t*>(smem + L.lvl());
    float* coef = reinterpret_cast<float*>(smem + L.coef());
    int32_t* cidx = reinterpret_cast<int32_t*>(smem + L.cidx());

    const int tid = threadIdx.x;
    const int b = blockIdx.x / a.Hv;
    const int h = blockIdx.x % a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const bool writer = (h == 0);   // one workgroup per tree publishes the tree

    // this tree's rows in the node arrays; the cache keeps N rows per tree
    const SeqRows rows = seq_rows(a.offsets, b, N);
    const int n = max(rows.n, 0);
    int status = tree_build_lds(a.parent + rows.row0, n, W, mask, jump, &s_flag);
    if (rows.n < 0) status = -1;

    // per-node base offsets in the documented layouts
    auto qk_off = [&](int i) { return ((rows.row0 + i) * a.Hk + hk) * dk; };
    auto v_off = [&](int i) { return ((rows.row0 + i) * a.Hv + h) * dv; };
    auto bg_off = [&](int i) { return (rows.row0 + i) * a.Hv + h; };
    float* U = a.u + ((size_t)b * a.Hv + h) * (size_t)N * dv;
    const float* S0 = a.S0 + ((size_t)b * a.Hv + h) * (size_t)dv * dk;

    if (writer) {
        uint32_t* gm = a.anc_mask + (size_t)b * N * W;
        for (int x = tid; x < N * W; x += kThreads) gm[x] = x < n * W ? mask[x] : 0u;
        for (int i = tid; i < N; i += kThreads)
            a.depth[(size_t)b * N + i] = (status || i >= n) ? -1 : row_popc(mask + i * W, W);
        if (tid == 0) a.status[b] = status;
    }
    if (status) {
        const float qnan = __uint_as_float(0x7fc00000u);
        for (int x = tid; x < N * dv; x += kThreads) {
            if (x < n * dv) st_io<IO>(a.o, v_off(x / dv) + x % dv, qnan);
            U[x] = qnan;
        }
        for (int i = tid; i < N; i += kThreads)
            a.log_gamma[((size_t)b * a.Hv + h) * N + i] = qnan;
        return;
    }

    // ln g per node, then G_i = sum of ln g over ancestors (ascending) + own.
    for (int i = tid; i < n; i += kThreads) lng[i] = logf(a.g[bg_off(i)]);
    if (tid == 0) s_maxdep = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
        const uint32_t* row = mask + i * W;
        float s = 0.f;
        int d = 0;
        for (int w = 0; w < W; ++w) {
            uint32_t x = row[w];
            d += __popc(x);
            while (x) {
                s += lng[w * 32 + __ffs(x) - 1];
                x &= x - 1u;
            }
        }
        lg[i] = s + lng[i];
        dep[i] = d;
        atomicMax(&s_maxdep, d);
        a.log_gamma[((size_t)b * a.Hv + h) * N + i] = lg[i];
    }
    __syncthreads();
    const int maxdep = s_maxdep;

    // Level-sorted node order (counting sort on depth).  The order inside a
    // level does not affect any value: every node's result depends only on its
    // own inputs and its ancestors' finished rows.
    for (int x = tid; x <= maxdep + 1; x += kThreads) lvl[x] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) atomicAdd(&lvl[dep[i] + 1], 1);
    __syncthreads();
    block_inclusive_scan(lvl, maxdep + 2, s_part);       // lvl[l] = first slot of level l
    for (int x = tid; x <= maxdep; x += kThreads) jump[x] = lvl[x];
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) order[atomicAdd(&jump[dep[i]], 1)] = i;
    __syncthreads();

    // Two sweeps over the levels: pass 0 solves (I + X) U = R, pass 1 forms O.
    // A chunk holds whole nodes whose coefficients fit kCoefCap; a node with
    // more coefficients than that is a chunk of its own and walks its ancestor
    // list in segments, carrying its fp32 partial sums in s_acc.
    for (int pass = 0; pass < 2; ++pass) {
        for (int l = 0; l <= maxdep; ++l) {
            const int beg = lvl[l], end = lvl[l + 1];
            const int per = pass == 0 ? l : l + 1;      // coefficients per node
            const int chunk = per > 0 ? max(1, kCoefCap / per) : max(1, end - beg);
            const int seg = max(1, min(per, kCoefCap));
            for (int c0 = beg; c0 < end; c0 += chunk) {
                const int c1 = min(end, c0 + chunk);
                const int nodes = c1 - c0;
                for (int m0 = 0; m0 == 0 || m0 < per; m0 += seg) {
                    const int mc = max(0, min(seg, per - m0));   // coefficients this segment
                    const bool first = m0 == 0, last = m0 + seg >= per;
                    for (int it = tid; it < nodes * mc; it += kThreads) {
                        const int i = order[c0 + it / mc];
                        const int m = m0 + it % mc;
                        const int j = (m < l) ? nth_set_bit(mask + i * W, W, m) : i;
                        const size_t oi = qk_off(i), oj = qk_off(j);
                        float dot = 0.f;
                        if (pass == 0) {
                            for (int c = 0; c < dk; ++c)
                                dot = fmaf(ld_io<IO>(a.k, oi + c), ld_io<IO>(a.k, oj + c), dot);
                            coef[it] = a.beta[bg_off(i)] * __expf(lg[i] - lg[j]) * dot;
                        } else {
                            for (int c = 0; c < dk; ++c)
                                dot = fmaf(ld_io<IO>(a.q, oi + c), ld_io<IO>(a.k, oj + c), dot);
                            coef[it] = __expf(lg[i] - lg[j]) * dot;
                        }
                        cidx[it] = j;
                    }
                    __syncthreads();
                    for (int it = tid; it < nodes * dv; it += kThreads) {
                        const int n = it / dv, r = it % dv;
                        const int i = order[c0 + n];
                        float acc;
                        if (first) {
                            const void* x = pass == 0 ? a.k : a.q;
                            const size_t oi = qk_off(i);
                            float sx = 0.f;                      // (S0 x_i)[r]
                            for (int c = 0; c < dk; ++c)
                                sx = fmaf(S0[(size_t)r * dk + c], ld_io<IO>(x, oi + c), sx);
                            const float eg = __expf(lg[i]);
                            acc = pass == 0 ? a.beta[bg_off(i)] * (ld_io<IO>(a.v, v_off(i) + r) - eg * sx)
                                            : eg * sx;
                        } else {
                            acc = s_acc[r];                      // one node per chunk here
                        }
                        const float sgn = pass == 0 ? -1.f : 1.f;
                        for (int m = 0; m < mc; ++m)
                            acc = fmaf(sgn * coef[n * mc + m], U[(size_t)cidx[n * mc + m] * dv + r], acc);
                        if (!last)
                            s_acc[r] = acc;
                        else if (pass == 0)
                            U[(size_t)i * dv + r] = acc;
                        else
                            st_io<IO>(a.o, v_off(i) + r, acc);
                    }
                    __syncthreads();
                }
            }
        }
    }
}

}  // namespace

size_t verify_generic_lds_bytes(int N) { return (size_t)GenericLds(N).words() * 4; }

hipError_t launch_verify_generic(const VerifyArgs& a, int io, hipStream_t stream) {
    const size_t lds = verify_generic_lds_bytes(a.N);
    // dynamic LDS plus the kernel's static LDS (two flags, s_part, s_acc:
    // 2056 bytes) must fit 160 KiB; 1024 nodes take 159748 + 2056
    constexpr size_t kStaticLds = 2 * sizeof(int) + kThreads * sizeof(int) + kMaxHead * sizeof(float);
    if (lds + kStaticLds > (size_t)kMaxLds) return hipErrorInvalidValue;
    const void* fn = io == GDN_BF16 ? (const void*)verify_generic_kernel<GDN_BF16>
                                    : (const void*)verify_generic_kernel<GDN_F32>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    VerifyArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(fn, dim3((unsigned)(a.B * a.Hv)), dim3(kThreads), args, lds,
                           stream);
}

}  // namespace gdn
