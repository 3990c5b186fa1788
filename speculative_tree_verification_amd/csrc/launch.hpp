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

// any tree of up to 1024 nodes (four nodes per thread past 256)
hipError_t launch_commit(const CommitArgs& a, bool bf16, hipStream_t stream);
// host-side checks of tree_ssd_commit_layers other than the table pointer;
// *nothing is set when the call has no work (no layers, items or nodes)
tsv_status check_commit_layers(const tsv_shape* s, int32_t n_layers, const int32_t* parent,
                               const int32_t* accepted, const int32_t* accepted_len, int32_t max_path_len,
                               bool* nothing);
// launch arguments of a multi-layer commit reading its table at `layers`
CommitArgs layers_args(const tsv_shape* s, int32_t n_layers, const tsv_commit_layer* layers,
                       const int32_t* parent, const int32_t* accepted, const int32_t* accepted_len,
                       int32_t max_path_len, int32_t* tree_status);

// trees of 257 to 1024 nodes: MFMA verify for bf16 with head_dim 64 and
// d_state 64 or 128, plain fp32 VALU verify otherwise (any P, N <= 256)
hipError_t launch_verify_large(const VerifyArgs& a, bool bf16, hipStream_t stream);

// gated delta rule over packed trees (q, k, v, o fp32 or bf16; T <= 64, dk and dv <= 128)
hipError_t launch_gdn_verify(int batch, int T, int H, int dk, int dv, bool bf16, const void* q,
                             const void* k, const void* v, const float* g, const float* beta,
                             const float* S0, const int32_t* parent, void* o, float* e,
                             int32_t* tree_status, hipStream_t stream);
// trees of 65 to 256 nodes (plain kernel; e is required: it holds the solve)
bool gdn_large_supported(int T);
hipError_t launch_gdn_large(int batch, int T, int H, int dk, int dv, bool bf16, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, const float* S0,
                            const int32_t* parent, void* o, float* e, int32_t* tree_status, hipStream_t stream);
// longest accepted path the gated-delta-rule commit takes past 64 nodes:
// the path's e and k rows are staged whole in LDS (up to 128 KiB)
constexpr int kGdnMaxPath = 128;
hipError_t launch_gdn_commit(int batch, int T, int H, int dk, int dv, bool bf16, const void* k,
                             const float* g, const float* e, float* S, const int32_t* parent,
                             const int32_t* accepted, const int32_t* accepted_len, int Lmax,
                             int32_t* tree_status, hipStream_t stream);

// ---- the forms a packed tree replaces (measured beside it)
struct UnrollArgs {
    const void* x;
    const void* dt;
    const void* B;
    const void* C;
    const float* h0;
    const int32_t* seq_nodes;
    const int32_t* seq_len;
    void* x_u;
    void* dt_u;
    void* B_u;
    void* C_u;
    float* h0_u;
    int batch, T, H, P, N, G, Lcap, S;
};
struct SeqScanArgs {
    const void* x_u;
    const void* dt_u;
    const float* A;
    const void* B_u;
    const void* C_u;
    const float* D;
    float* h_io;
    const int32_t* seq_len;
    void* y_u;
    int nseq, S, H, P, N, G;
};
hipError_t launch_unroll_plan(int batch, int T, const int32_t* parent, int Lcap, int S, int32_t* seq_nodes,
                              int32_t* seq_len, int32_t* n_leaves, int32_t* tree_status, hipStream_t stream);
hipError_t launch_unroll_gather(const UnrollArgs& u, bool bf16, hipStream_t stream);
hipError_t launch_seq_scan(const SeqScanArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_snapshot_verify(const VerifyArgs& a, float* states, bool bf16, hipStream_t stream);
hipError_t launch_snapshot_commit(int batch, int T, int H, int PN, const float* states, float* h0,
                                  const int32_t* parent, const int32_t* accepted,
                                  const int32_t* accepted_len, int Lmax, int32_t* tree_status,
                                  hipStream_t stream);

// greedy acceptance of a verified tree (one work-group per item)
hipError_t launch_accept_greedy(int batch, int T, const int32_t* parent, const int32_t* draft,
                                const int32_t* target, int Lmax, int32_t* accepted,
                                int32_t* accepted_len, int32_t* next_token, int32_t* tree_status,
                                hipStream_t stream);
hipError_t launch_accept_stochastic(int batch, int T, int V, const int32_t* parent, const int32_t* draft,
                                    const float* p_target, const float* q_draft, const float* u_node,
                                    const float* u_final, int Lmax, int32_t* accepted, int32_t* accepted_len,
                                    int32_t* next_token, int32_t* tree_status, hipStream_t stream);

}  // namespace tsv
