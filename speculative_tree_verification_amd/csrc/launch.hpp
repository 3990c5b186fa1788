// launch.hpp -- host-side launchers of the tree-SSD kernels (one per .hip file).
// Shapes are validated by the C-ABI layer (api.hip) before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tree_ssd.h"

namespace tsv {

struct VerifyArgs {
    const void* x;
    const void* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* h0;
    const int32_t* parent;
    void* y;
    int32_t* tree_status;
    int batch, T, H, P, N, G;
};

// One layer's operands (x, dt, A, B, h), or, with `layers` set, a device table
// of n_layers of them (the five direct pointers are then unused).
struct CommitArgs {
    const void* x;
    const void* dt;
    const float* A;
    const void* B;
    float* h;
    const tsv_commit_layer* layers;
    int n_layers;
    const int32_t* parent;
    const int32_t* accepted;
    const int32_t* accepted_len;
    int32_t* tree_status;
    int batch, T, H, P, N, G, Lmax;
};

hipError_t launch_tree_info(int batch, int T, const int32_t* parent, int32_t* depth,
                            uint64_t* anc, int32_t* tree_status, hipStream_t stream);

// plain VALU verify, any P, N <= 256; bf16 selects the bf16 input dtype
hipError_t launch_verify_generic(const VerifyArgs& a, bool bf16, hipStream_t stream);

// bf16 MFMA verify (head_dim 64, d_state 64 or 128): trees of <= 64 nodes use
// the per-wave head_dim-slice kernel, wider trees the LDS-staged kernel
hipError_t launch_verify_small(const VerifyArgs& a, int heads_per_block, hipStream_t stream);
hipError_t launch_verify_wide(const VerifyArgs& a, int heads_per_block, hipStream_t stream);
// bf16 MFMA verify for trees of at most 16 nodes: one wave per (item, head,
// 16-row slice of head_dim), no LDS, no barrier (heads_per_block does not apply)
hipError_t launch_verify_tiny(const VerifyArgs& a, hipStream_t stream);

hipError_t launch_commit(const CommitArgs& a, bool bf16, hipStream_t stream);

// trees of 257 to 1024 nodes: plain fp32 VALU verify and commit (any P, N <= 256)
hipError_t launch_verify_large(const VerifyArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_commit_large(const CommitArgs& a, bool bf16, hipStream_t stream);

// gated delta rule over packed trees (fp32, T <= 64, dk and dv <= 128)
hipError_t launch_gdn_verify(int batch, int T, int H, int dk, int dv, const float* q,
                             const float* k, const float* v, const float* g, const float* beta,
                             const float* S0, const int32_t* parent, float* o, float* e,
                             int32_t* tree_status, hipStream_t stream);
hipError_t launch_gdn_commit(int batch, int T, int H, int dk, int dv, const float* k,
                             const float* g, const float* e, float* S, const int32_t* parent,
                             const int32_t* accepted, const int32_t* accepted_len, int Lmax,
                             int32_t* tree_status, hipStream_t stream);

// greedy acceptance of a verified tree (one work-group per item)
hipError_t launch_accept_greedy(int batch, int T, const int32_t* parent, const int32_t* draft,
                                const int32_t* target, int Lmax, int32_t* accepted,
                                int32_t* accepted_len, int32_t* next_token, int32_t* tree_status,
                                hipStream_t stream);

}  // namespace tsv
