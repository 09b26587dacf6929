// abi.hip -- the library's C ABI: argument checks, kernel selection, launches.
// Every check runs on the host before anything is enqueued; a failed check
// returns a negative gdn_status and launches nothing.
#include <stdint.h>

#include "gdn_common.hpp"
#include "launch.hpp"

namespace {

using namespace gdn;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_dims(const gdn_tree_dims* d) {
    if (!d) return GDN_ERR_NULL;
    if (d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (d->batch < 0 || d->n_nodes < 1 || d->n_nodes > kMaxNodes) return GDN_ERR_DIMS;
    if (d->h_k < 1 || d->h_v < 1 || d->h_v % d->h_k != 0) return GDN_ERR_DIMS;
    if (d->d_k < 1 || d->d_k > kMaxHead || d->d_v < 1 || d->d_v > kMaxHead)
        return GDN_ERR_DIMS;
    // the grid's x extent is batch * h_v workgroups
    if ((int64_t)d->batch * d->h_v > 0x7fffffffLL) return GDN_ERR_DIMS;
    return GDN_OK;
}

int check_cache(const gdn_tree_cache* c) {
    if (!c || !c->anc_mask || !c->depth || !c->u || !c->log_gamma || !c->tree_status)
        return GDN_ERR_NULL;
    if (misaligned(c->anc_mask) || misaligned(c->depth) || misaligned(c->u) ||
        misaligned(c->log_gamma) || misaligned(c->tree_status))
        return GDN_ERR_ALIGN;
    return GDN_OK;
}

// offsets: nullptr for the dense layout, else the ragged layout's first rows
int verify_impl(const gdn_tree_dims* dims, const int32_t* offsets, const float* S0, const void* q,
                const void* k, const void* v, const float* beta, const float* g,
                const int32_t* parent, void* o, const gdn_tree_cache* cache, hipStream_t stream) {
    if (!S0 || !q || !k || !v || !beta || !g || !parent || !o) return GDN_ERR_NULL;
    int rc = check_cache(cache);
    if (rc) return rc;
    if (misaligned(S0) || misaligned(q) || misaligned(k) || misaligned(v) ||
        misaligned(beta) || misaligned(g) || misaligned(parent) || misaligned(o))
        return GDN_ERR_ALIGN;

    VerifyArgs a{dims->batch, dims->n_nodes, dims->h_k, dims->h_v, dims->d_k, dims->d_v,
                 S0, q, k, v, beta, g, parent, o,
                 cache->anc_mask, cache->depth, cache->u, cache->log_gamma,
                 cache->tree_status, offsets};
    hipError_t e = verify_tiled_supported(a, dims->io_dtype)   ? launch_verify_tiled(a, dims->io_dtype, stream)
                   : verify_large_supported(a, dims->io_dtype) ? launch_verify_large(a, dims->io_dtype, stream)
                                                               : launch_verify_generic(a, dims->io_dtype, stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int commit_impl(const gdn_tree_dims* dims, const int32_t* offsets, const float* S_in, float* S_out,
                const void* k, const gdn_tree_cache* cache, const int32_t* accepted,
                int32_t* path, int32_t* path_len, hipStream_t stream) {
    if (!S_in || !S_out || !k || !accepted || !path || !path_len) return GDN_ERR_NULL;
    int rc = check_cache(cache);
    if (rc) return rc;
    if (misaligned(S_in) || misaligned(S_out) || misaligned(k) || misaligned(accepted) ||
        misaligned(path) || misaligned(path_len))
        return GDN_ERR_ALIGN;

    CommitArgs a{dims->batch, dims->n_nodes, dims->h_k, dims->h_v, dims->d_k, dims->d_v,
                 S_in, S_out, k, cache->anc_mask, cache->u, cache->log_gamma,
                 cache->tree_status, accepted, path, path_len, offsets};
    hipError_t e = launch_commit(a, dims->io_dtype, stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int commit_verify_impl(const gdn_tree_dims* dims, const int32_t* offsets_prev, const float* S_prev,
                       float* S_new, const void* k_prev, const gdn_tree_cache* cache_prev,
                       const int32_t* accepted_prev, int32_t* path_prev, int32_t* path_len_prev,
                       const int32_t* offsets, const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const int32_t* parent, void* o,
                       const gdn_tree_cache* cache, hipStream_t stream) {
    if (!S_prev || !S_new || !k_prev || !accepted_prev || !path_prev || !path_len_prev || !q || !k ||
        !v || !beta || !g || !parent || !o)
        return GDN_ERR_NULL;
    int rc = check_cache(cache_prev);
    if (rc) return rc;
    rc = check_cache(cache);
    if (rc) return rc;
    if (misaligned(S_prev) || misaligned(S_new) || misaligned(k_prev) || misaligned(accepted_prev) ||
        misaligned(path_prev) || misaligned(path_len_prev) || misaligned(q) || misaligned(k) ||
        misaligned(v) || misaligned(beta) || misaligned(g) || misaligned(parent) || misaligned(o))
        return GDN_ERR_ALIGN;
    const void* prev_bufs[] = {cache_prev->anc_mask, cache_prev->depth, cache_prev->u,
                               cache_prev->log_gamma, cache_prev->tree_status};
    const void* new_bufs[] = {cache->anc_mask, cache->depth, cache->u, cache->log_gamma,
                              cache->tree_status};
    for (const void* x : prev_bufs)
        for (const void* y : new_bufs)
            if (x == y) return GDN_ERR_ALIAS;

    CommitArgs c{dims->batch, dims->n_nodes, dims->h_k, dims->h_v, dims->d_k, dims->d_v,
                 S_prev, S_new, k_prev, cache_prev->anc_mask, cache_prev->u, cache_prev->log_gamma,
                 cache_prev->tree_status, accepted_prev, path_prev, path_len_prev, offsets_prev};
    VerifyArgs a{dims->batch, dims->n_nodes, dims->h_k, dims->h_v, dims->d_k, dims->d_v,
                 S_prev, q, k, v, beta, g, parent, o,
                 cache->anc_mask, cache->depth, cache->u, cache->log_gamma,
                 cache->tree_status, offsets};
    hipError_t e;
    if (verify_tiled_supported(a, dims->io_dtype)) {
        e = launch_commit_verify_tiled(a, c, dims->io_dtype, stream);
    } else if (verify_large_supported(a, dims->io_dtype)) {
        e = launch_commit_verify_large(a, c, dims->io_dtype, stream);
    } else {
        e = launch_commit(c, dims->io_dtype, stream);
        if (e == hipSuccess) {
            a.S0 = S_new;
            e = launch_verify_generic(a, dims->io_dtype, stream);
        }
    }
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int accept_impl(const gdn_tree_dims* dims, const int32_t* offsets, const int32_t* parent,
                const int32_t* draft, const int32_t* target, const int32_t* target_root,
                int32_t* accepted, int32_t* accept_len, int32_t* next_token, hipStream_t stream) {
    if (!parent || !draft || !target || !target_root || !accepted || !accept_len || !next_token)
        return GDN_ERR_NULL;
    if (misaligned(parent) || misaligned(draft) || misaligned(target) || misaligned(target_root) ||
        misaligned(accepted) || misaligned(accept_len) || misaligned(next_token))
        return GDN_ERR_ALIGN;
    AcceptArgs a{dims->batch, dims->n_nodes, parent, draft, target, target_root,
                 accepted, accept_len, next_token, offsets};
    return launch_accept(a, stream) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// A ragged call's offsets array: present and int32-aligned.
int check_offsets(const int32_t* offsets) {
    if (!offsets) return GDN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(offsets) & 3u) != 0) return GDN_ERR_ALIGN;
    return GDN_OK;
}

}  // namespace

extern "C" {


int gdn_tree_cache_bytes(const gdn_tree_dims* dims, size_t* anc_mask, size_t* depth,
                         size_t* u, size_t* log_gamma, size_t* tree_status) {
    int rc = check_dims(dims);
    if (rc) return rc;
    const size_t B = dims->batch, N = dims->n_nodes, W = (N + 31) / 32;
    if (anc_mask) *anc_mask = B * N * W * sizeof(uint32_t);
    if (depth) *depth = B * N * sizeof(int32_t);
    if (u) *u = B * (size_t)dims->h_v * N * (size_t)dims->d_v * sizeof(float);
    if (log_gamma) *log_gamma = B * (size_t)dims->h_v * N * sizeof(float);
    if (tree_status) *tree_status = B * sizeof(int32_t);
    return GDN_OK;
}

int gdn_tree_verify(const gdn_tree_dims* dims, const float* S0, const void* q,
                    const void* k, const void* v, const float* beta, const float* g,
                    const int32_t* parent, void* o, const gdn_tree_cache* cache,
                    hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->batch == 0) return GDN_OK;
    return verify_impl(dims, nullptr, S0, q, k, v, beta, g, parent, o, cache, stream);
}

int gdn_tree_verify_ragged(const gdn_tree_dims* dims, const int32_t* offsets, const float* S0,
                           const void* q, const void* k, const void* v, const float* beta,
                           const float* g, const int32_t* parent, void* o,
                           const gdn_tree_cache* cache, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->batch == 0) return GDN_OK;
    rc = check_offsets(offsets);
    if (rc) return rc;
    return verify_impl(dims, offsets, S0, q, k, v, beta, g, parent, o, cache, stream);
}

int gdn_tree_commit(const gdn_tree_dims* dims, const float* S_in, float* S_out,
                    const void* k, const gdn_tree_cache* cache, const int32_t* accepted,
                    int32_t* path, int32_t* path_len, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->batch == 0) return GDN_OK;
    return commit_impl(dims, nullptr, S_in, S_out, k, cache, accepted, path, path_len, stream);
}

int gdn_tree_commit_ragged(const gdn_tree_dims* dims, const int32_t* offsets, const float* S_in,
                           float* S_out, const void* k, const gdn_tree_cache* cache,
                           const int32_t* accepted, int32_t* path, int32_t* path_len,
                           hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->batch == 0) return GDN_OK;
    rc = check_offsets(offsets);
    if (rc) return rc;
    return commit_impl(dims, offsets, S_in, S_out, k, cache, accepted, path, path_len, stream);
}

int gdn_tree_commit_verify(const gdn_tree_dims* dims, const float* S_prev, float* S_new,
                           const void* k_prev, const gdn_tree_cache* cache_prev,
                           const int32_t* accepted_prev, int32_t* path_prev,
                           int32_t* path_len_prev, const void* q, const void* k,
                           const void* v, const float* beta, const float* g,
                           const int32_t* parent, void* o, const gdn_tree_cache* cache,
                           hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->batch == 0) return GDN_OK;
    return commit_verify_impl(dims, nullptr, S_prev, S_new, k_prev, cache_prev, accepted_prev,
                              path_prev, path_len_prev, nullptr, q, k, v, beta, g, parent, o,
                              cache, stream);
}

int gdn_tree_commit_verify_ragged(const gdn_tree_dims* dims, const int32_t* offsets_prev,
                                  const float* S_prev, float* S_new, const void* k_prev,
                                  const gdn_tree_cache* cache_prev, const int32_t* accepted_prev,
                                  int32_t* path_prev, int32_t* path_len_prev,
                                  const int32_t* offsets, const void* q, const void* k,
                                  const void* v, const float* beta, const float* g,
                                  const int32_t* parent, void* o, const gdn_tree_cache* cache,
                                  hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->batch == 0) return GDN_OK;
    rc = check_offsets(offsets_prev);
    if (rc) return rc;
    rc = check_offsets(offsets);
    if (rc) return rc;
    return commit_verify_impl(dims, offsets_prev, S_prev, S_new, k_prev, cache_prev, accepted_prev,
                              path_prev, path_len_prev, offsets, q, k, v, beta, g, parent, o,
                              cache, stream);
}

int gdn_tree_accept(const gdn_tree_dims* dims, const int32_t* parent, const int32_t* draft,
                    const int32_t* target, const int32_t* target_root, int32_t* accepted,
                    int32_t* accept_len, int32_t* next_token, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->batch == 0) return GDN_OK;
    return accept_impl(dims, nullptr, parent, draft, target, target_root, accepted, accept_len,
                       next_token, stream);
}

int gdn_tree_accept_ragged(const gdn_tree_dims* dims, const int32_t* offsets, const int32_t* parent,
                           const int32_t* draft, const int32_t* target, const int32_t* target_root,
                           int32_t* accepted, int32_t* accept_len, int32_t* next_token,
                           hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->batch == 0) return GDN_OK;
    rc = check_offsets(offsets);
    if (rc) return rc;
    return accept_impl(dims, offsets, parent, draft, target, target_root, accepted, accept_len,
                       next_token, stream);
}

int gdn_tree_build(const gdn_tree_build_dims* dims, const float* logp, const int32_t* tok,
                   int32_t* parent, int32_t* token, float* score, hipStream_t stream) {
    if (!dims) return GDN_ERR_NULL;
    if (dims->batch < 0 || dims->n_nodes < 1 || dims->n_nodes > kMaxNodes || dims->topk < 1 ||
        dims->topk > kMaxBuildTopk || dims->width < 1)
        return GDN_ERR_DIMS;
    if (tree_build_lds_bytes(dims->n_nodes, dims->topk, dims->width) > (size_t)kMaxLds)
        return GDN_ERR_DIMS;
    if (dims->batch == 0) return GDN_OK;
    if (!logp || !tok || !parent || !token || !score) return GDN_ERR_NULL;
    if (misaligned(logp) || misaligned(tok) || misaligned(parent) || misaligned(token) ||
        misaligned(score))
        return GDN_ERR_ALIGN;
    BuildArgs a{dims->batch, dims->n_nodes, dims->topk, dims->width, logp, tok, parent, token, score};
    return launch_tree_build(a, stream) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

const char* gdn_tree_strerror(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_DIMS: return "sizes outside the supported range";
        case GDN_ERR_DTYPE: return "io_dtype is not GDN_F32 or GDN_BF16";
        case GDN_ERR_LAUNCH: return "a kernel launch failed";
        case GDN_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
        case GDN_ERR_ALIAS: return "two caches that must be distinct share a buffer";
        default: return "unknown gdn_status";
    }
}

}  // extern "C"
