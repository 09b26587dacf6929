// launch.hpp -- host-side launchers of the library's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_common.hpp"

namespace gdn {

// General-shape verification: any valid size, fp32 vector arithmetic.
size_t verify_generic_lds_bytes(int n_nodes);
hipError_t launch_verify_generic(const VerifyArgs& a, int io, hipStream_t stream);

// MFMA verification: d_k = d_v = 128, bf16 io, up to 128 nodes.
bool verify_tiled_supported(const VerifyArgs& a, int io);
hipError_t launch_verify_tiled(const VerifyArgs& a, int io, hipStream_t stream);
// The same with the previous tree's commit fused in front (a.S0 = c.S_in).
hipError_t launch_commit_verify_tiled(const VerifyArgs& a, const CommitArgs& c, int io, hipStream_t stream);

// MFMA verification of larger trees: d_k = d_v = 128, bf16 io, 129 .. 512 nodes
// (one launch: the tree check, its ancestor rows into the cache, the solve).
bool verify_large_supported(const VerifyArgs& a, int io);
hipError_t launch_verify_large(const VerifyArgs& a, int io, hipStream_t stream);
// The same with the previous tree's commit fused in front (a.S0 = c.S_in).
hipError_t launch_commit_verify_large(const VerifyArgs& a, const CommitArgs& c, int io, hipStream_t stream);

// Deferred commit of the accepted node's state.
hipError_t launch_commit(const CommitArgs& a, int io, hipStream_t stream);

// Greedy acceptance walk, one wave per sequence.
struct AcceptArgs {
    int B, N;
    const int32_t* parent;
    const int32_t* draft;
    const int32_t* target;
    const int32_t* target_root;
    int32_t* accepted;
    int32_t* accept_len;
    int32_t* next_token;
    const int32_t* offsets;   // ragged layout: [B + 1] first rows; nullptr = dense
};
hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream);

// Draft-tree construction with w expansions per step, one wave per sequence.
constexpr int kMaxBuildTopk = 64;   // continuations per drafter row
struct BuildArgs {
    int B, N, K, w;
    const float* logp;        // [B][N + 1][K]
    const int32_t* tok;       // [B][N + 1][K]
    int32_t* parent;          // [B][N]
    int32_t* token;           // [B][N]
    float* score;             // [B][N]
};
size_t tree_build_lds_bytes(int N, int K, int w);
hipError_t launch_tree_build(const BuildArgs& a, hipStream_t stream);

}  // namespace gdn
