// api.hip -- extern "C" entry points of libtree_ssd.so (declared in
// include/tree_ssd.h). Host-side validation happens here, before anything is
// enqueued; the kernels themselves only see consistent shapes.
#include "tree_ssd.h"
#include "launch.hpp"

namespace {

constexpr int kMaxNodes = 1024;  // trees past 256 nodes take the plain kernels
constexpr int kMaxNodesMfma = 256;
constexpr int kMaxDim = 256;

tsv_status check_shape(const tsv_shape* s) {
    if (!s) return TSV_E_NULL;
    if (s->in_dtype != TSV_F32 && s->in_dtype != TSV_BF16) return TSV_E_DTYPE;
    if (s->batch < 0 || s->n_nodes < 0 || s->n_nodes > kMaxNodes) return TSV_E_SHAPE;
    if (s->n_heads < 1 || s->head_dim < 1 || s->d_state < 1 || s->n_groups < 1) return TSV_E_SHAPE;
    if (s->n_heads % s->n_groups != 0) return TSV_E_SHAPE;
    if (s->heads_per_block < 0) return TSV_E_SHAPE;
    if (s->heads_per_block > 0 && (s->n_heads / s->n_groups) % s->heads_per_block != 0)
        return TSV_E_SHAPE;
    if (s->head_dim > kMaxDim || s->d_state > kMaxDim) return TSV_E_UNSUPPORTED;
    if (s->n_heads > 0xffff) return TSV_E_UNSUPPORTED;  // sizes are packed into 16-bit fields
    // the per-launch grid stays well inside 2^31 work-groups
    if ((long long)s->batch * s->n_heads * 64 > 0x7fffffffLL) return TSV_E_UNSUPPORTED;
    return TSV_OK;
}

bool use_mfma(const tsv_shape* s) {
    return s->in_dtype == TSV_BF16 && !(s->flags & TSV_FLAG_FORCE_GENERIC) &&
           s->n_nodes <= kMaxNodesMfma && s->head_dim == 64 && (s->d_state == 64 || s->d_state == 128);
}

int compute_units() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

// Heads per work-group: the largest divisor of the heads of one group that
// still gives the GPU `per_cu` work-groups per compute unit. More heads per
// work-group amortise the tree set-up (validation, pair lists, pair scores);
// fewer leave more work-groups to hide memory latency. Measured on the
// batched Mamba2-2.7B and 8B-hybrid shapes: the small-tree kernel (which
// computes a work-group's heads side by side) does best at four work-groups
// per compute unit, the wide-tree kernel (which fills a compute unit's LDS
// and takes its heads one after another) at one.
int default_heads_per_block(const tsv_shape* s, int per_cu) {
    const long want = (long)compute_units() * per_cu;
    const int hpg = s->n_heads / s->n_groups;
    int best = 1;
    for (int d = 1; d <= hpg; ++d)
        if (hpg % d == 0 && (long)s->batch * (s->n_heads / d) >= want) best = d;
    return best;
}
hipError_t launch_mfma(const tsv_shape* s, const tsv::VerifyArgs& a, hipStream_t hs) {
    if (s->n_nodes <= 16 && !(s->flags & (TSV_FLAG_FORCE_WIDE | TSV_FLAG_FORCE_SMALL)))
        return tsv::launch_verify_tiny(a, hs);
    const bool small = s->n_nodes <= 64 && !(s->flags & TSV_FLAG_FORCE_WIDE);
    int hb = s->heads_per_block;
    if (hb == 0) hb = default_heads_per_block(s, small ? 4 : 1);
    return small ? tsv::launch_verify_small(a, hb, hs) : tsv::launch_verify_wide(a, hb, hs);
}
}  // namespace

extern "C" {

tsv_status tree_ssd_verify(const tsv_shape* s, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, const float* h0,
                           const int32_t* parent, void* y, int32_t* tree_status, void* stream) {
    tsv_status st = check_shape(s);
    if (st != TSV_OK) return st;
    if (s->batch == 0 || s->n_nodes == 0) return TSV_OK;
    if (!x || !dt || !A || !B || !C || !D || !h0 || !parent || !y) return TSV_E_NULL;
    tsv::VerifyArgs a{x,  dt, A,           B,        C,          D,          h0,
                      parent, y, tree_status, s->batch, s->n_nodes, s->n_heads, s->head_dim,
                      s->d_state, s->n_groups};
    hipStream_t hs = (hipStream_t)stream;
    const bool bf16 = s->in_dtype == TSV_BF16;
    hipError_t e = s->n_nodes > kMaxNodesMfma ? tsv::launch_verify_large(a, bf16, hs)
                   : use_mfma(s)             ? launch_mfma(s, a, hs)
                                             : tsv::launch_verify_generic(a, bf16, hs);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_ssd_commit(const tsv_shape* s, const void* x, const void* dt, const float* A,
                           const void* B, float* h0_inout, const int32_t* parent,
                           const int32_t* accepted, const int32_t* accepted_len,
                           int32_t max_path_len, int32_t* tree_status, void* stream) {
    tsv_status st = check_shape(s);
    if (st != TSV_OK) return st;
    if (max_path_len < 0 || max_path_len > kMaxNodes) return TSV_E_SHAPE;
    if (s->batch == 0 || s->n_nodes == 0) return TSV_OK;
    if (!x || !dt || !A || !B || !h0_inout || !parent || !accepted_len) return TSV_E_NULL;
    if (max_path_len > 0 && !accepted) return TSV_E_NULL;
    tsv::CommitArgs a{x,        dt,          A,           B,           h0_inout,   nullptr,
                      1,        parent,      accepted,    accepted_len, tree_status, s->batch,
                      s->n_nodes, s->n_heads, s->head_dim, s->d_state,  s->n_groups, max_path_len};
    hipError_t e = tsv::launch_commit(a, s->in_dtype == TSV_BF16, (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_ssd_commit_layers(const tsv_shape* s, int32_t n_layers,
                                  const tsv_commit_layer* layers, const int32_t* parent,
                                  const int32_t* accepted, const int32_t* accepted_len,
                                  int32_t max_path_len, int32_t* tree_status, void* stream) {
    bool nothing = false;
    tsv_status st = tsv::check_commit_layers(s, n_layers, parent, accepted, accepted_len, max_path_len, &nothing);
    if (st != TSV_OK || nothing) return st;
    if (!layers) return TSV_E_NULL;
    hipError_t e = tsv::launch_commit(tsv::layers_args(s, n_layers, layers, parent, accepted, accepted_len,
                                                       max_path_len, tree_status),
                                      s->in_dtype == TSV_BF16, (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

}  // extern "C"

namespace tsv {

tsv_status check_commit_layers(const tsv_shape* s, int32_t n_layers, const int32_t* parent,
                               const int32_t* accepted, const int32_t* accepted_len, int32_t max_path_len,
                               bool* nothing) {
    *nothing = false;
    tsv_status st = check_shape(s);
    if (st != TSV_OK) return st;
    if (n_layers < 0 || max_path_len < 0 || max_path_len > kMaxNodes) return TSV_E_SHAPE;
    if (n_layers == 0 || s->batch == 0 || s->n_nodes == 0) {
        *nothing = true;
        return TSV_OK;
    }
    if (!parent || !accepted_len) return TSV_E_NULL;
    if (max_path_len > 0 && !accepted) return TSV_E_NULL;
    // the grid (layers x items x heads x state chunks) stays inside 2^31 work-groups
    if ((long long)n_layers * s->batch * s->n_heads * 64 > 0x7fffffffLL) return TSV_E_UNSUPPORTED;
    return TSV_OK;
}

CommitArgs layers_args(const tsv_shape* s, int32_t n_layers, const tsv_commit_layer* layers,
                       const int32_t* parent, const int32_t* accepted, const int32_t* accepted_len,
                       int32_t max_path_len, int32_t* tree_status) {
    return CommitArgs{nullptr,  nullptr,     nullptr,     nullptr,      nullptr,     layers,
                      n_layers, parent,      accepted,    accepted_len, tree_status, s->batch,
                      s->n_nodes, s->n_heads, s->head_dim, s->d_state,  s->n_groups, max_path_len};
}

}  // namespace tsv

extern "C" {

namespace {
// gated-delta-rule shapes: fp32, one group, T <= 64, dk = d_state and
// dv = head_dim up to 128
tsv_status check_gdn_shape(const tsv_shape* s) {
    tsv_status st = check_shape(s);
    if (st != TSV_OK) return st;
    if ((s->in_dtype != TSV_F32 && s->in_dtype != TSV_BF16) || s->n_groups != 1) return TSV_E_UNSUPPORTED;
    if (s->n_nodes > kMaxNodesMfma || s->head_dim > 128 || s->d_state > 128) return TSV_E_UNSUPPORTED;
    return TSV_OK;
}
}  // namespace

tsv_status tree_gdn_verify(const tsv_shape* s, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const float* S0,
                           const int32_t* parent, void* o, float* e, int32_t* tree_status,
                           void* stream) {
    tsv_status st = check_gdn_shape(s);
    if (st != TSV_OK) return st;
    if (s->batch == 0 || s->n_nodes == 0) return TSV_OK;
    if (!q || !k || !v || !g || !beta || !S0 || !parent || !o) return TSV_E_NULL;
    if (tsv::gdn_large_supported(s->n_nodes)) {
        hipError_t err = tsv::launch_gdn_large(s->batch, s->n_nodes, s->n_heads, s->d_state, s->head_dim,
                                               s->in_dtype == TSV_BF16, q, k, v, g, beta, S0, parent, o, e,
                                               tree_status, (hipStream_t)stream);
        return err == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
    }
    hipError_t err = tsv::launch_gdn_verify(s->batch, s->n_nodes, s->n_heads, s->d_state,
                                            s->head_dim, s->in_dtype == TSV_BF16, q, k, v, g, beta,
                                            S0, parent, o, e,
                                            tree_status, (hipStream_t)stream);
    return err == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_gdn_commit(const tsv_shape* s, const void* k, const float* g, const float* e,
                           float* S0_inout, const int32_t* parent, const int32_t* accepted,
                           const int32_t* accepted_len, int32_t max_path_len, int32_t* tree_status,
                           void* stream) {
    tsv_status st = check_gdn_shape(s);
    if (st != TSV_OK) return st;
    if (max_path_len < 0 || max_path_len > kMaxNodes) return TSV_E_SHAPE;
    if (s->n_nodes > 64 && max_path_len > tsv::kGdnMaxPath) return TSV_E_UNSUPPORTED;  // paths staged whole in LDS
    if (s->batch == 0 || s->n_nodes == 0) return TSV_OK;
    if (!k || !g || !e || !S0_inout || !parent || !accepted_len) return TSV_E_NULL;
    if (max_path_len > 0 && !accepted) return TSV_E_NULL;
    hipError_t err = tsv::launch_gdn_commit(s->batch, s->n_nodes, s->n_heads, s->d_state,
                                            s->head_dim, s->in_dtype == TSV_BF16, k, g, e, S0_inout,
                                            parent, accepted,
                                            accepted_len, max_path_len, tree_status,
                                            (hipStream_t)stream);
    return err == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_ssd_accept_greedy(int32_t batch, int32_t n_nodes, const int32_t* parent,
                                  const int32_t* draft_tokens, const int32_t* target_tokens,
                                  int32_t max_path_len, int32_t* accepted, int32_t* accepted_len,
                                  int32_t* next_token, int32_t* tree_status, void* stream) {
    if (batch < 0 || n_nodes < 0 || n_nodes > kMaxNodes) return TSV_E_SHAPE;
    if (max_path_len < 1 || max_path_len > kMaxNodes) return TSV_E_SHAPE;
    if (batch == 0 || n_nodes == 0) return TSV_OK;
    if (!parent || !draft_tokens || !target_tokens || !accepted || !accepted_len) return TSV_E_NULL;
    hipError_t e = tsv::launch_accept_greedy(batch, n_nodes, parent, draft_tokens, target_tokens,
                                             max_path_len, accepted, accepted_len, next_token,
                                             tree_status, (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_ssd_accept_stochastic(int32_t batch, int32_t n_nodes, int32_t vocab,
                                      const int32_t* parent, const int32_t* draft_tokens,
                                      const float* p_target, const float* q_draft, const float* u_node,
                                      const float* u_final, int32_t max_path_len, int32_t* accepted,
                                      int32_t* accepted_len, int32_t* next_token, int32_t* tree_status,
                                      void* stream) {
    if (batch < 0 || n_nodes < 0 || n_nodes > kMaxNodes || vocab < 1) return TSV_E_SHAPE;
    if (max_path_len < 1 || max_path_len > kMaxNodes) return TSV_E_SHAPE;
    if (batch == 0 || n_nodes == 0) return TSV_OK;
    if (!parent || !draft_tokens || !p_target || !q_draft || !u_node || !u_final || !accepted ||
        !accepted_len)
        return TSV_E_NULL;
    hipError_t e = tsv::launch_accept_stochastic(batch, n_nodes, vocab, parent, draft_tokens, p_target,
                                                 q_draft, u_node, u_final, max_path_len, accepted,
                                                 accepted_len, next_token, tree_status, (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_ssd_tree_info(int32_t batch, int32_t n_nodes, const int32_t* parent,
                              int32_t* depth, uint64_t* anc_bits, int32_t* tree_status,
                              void* stream) {
    if (batch < 0 || n_nodes < 0 || n_nodes > kMaxNodes) return TSV_E_SHAPE;
    if (batch == 0 || n_nodes == 0) return TSV_OK;
    if (!parent || !depth || !anc_bits) return TSV_E_NULL;
    hipError_t e = tsv::launch_tree_info(batch, n_nodes, parent, depth, anc_bits, tree_status,
                                         (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

// ---- the forms a packed tree replaces
namespace {
constexpr int kBaseMaxDim = 256;     // head_dim, d_state of the baseline kernels
constexpr int kBaseMaxState = 16384; // head_dim * d_state: 64 state elements per thread
}  // namespace

tsv_status tree_ssd_unroll_plan(int32_t batch, int32_t n_nodes, const int32_t* parent, int32_t max_leaves,
                                int32_t max_len, int32_t* seq_nodes, int32_t* seq_len, int32_t* n_leaves,
                                int32_t* tree_status, void* stream) {
    if (batch < 0 || n_nodes < 0 || n_nodes > kMaxNodes) return TSV_E_SHAPE;
    if (max_leaves < 1 || max_leaves > kMaxNodes || max_len < 1 || max_len > kMaxNodes) return TSV_E_SHAPE;
    if (batch == 0 || n_nodes == 0) return TSV_OK;
    if (!parent || !seq_nodes || !seq_len || !n_leaves) return TSV_E_NULL;
    hipError_t e = tsv::launch_unroll_plan(batch, n_nodes, parent, max_leaves, max_len, seq_nodes, seq_len,
                                           n_leaves, tree_status, (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_ssd_unroll_gather(const tsv_shape* s, int32_t max_leaves, int32_t max_len, const void* x,
                                  const void* dt, const void* B, const void* C, const float* h0,
                                  const int32_t* seq_nodes, const int32_t* seq_len, void* x_u, void* dt_u,
                                  void* B_u, void* C_u, float* h0_u, void* stream) {
    tsv_status st = check_shape(s);
    if (st != TSV_OK) return st;
    if (max_leaves < 1 || max_leaves > kMaxNodes || max_len < 1 || max_len > kMaxNodes) return TSV_E_SHAPE;
    if (s->batch == 0 || s->n_nodes == 0) return TSV_OK;
    if (!x || !dt || !B || !C || !h0 || !seq_nodes || !seq_len || !x_u || !dt_u || !B_u || !C_u || !h0_u)
        return TSV_E_NULL;
    const long long nseq = (long long)s->batch * max_leaves;
    if (nseq * (max_len + s->n_heads) > 0x7fffffffLL) return TSV_E_UNSUPPORTED;
    tsv::UnrollArgs u{x,  dt,   B,    C,        h0,       seq_nodes,   seq_len,    x_u,
                      dt_u, B_u, C_u, h0_u, s->batch, s->n_nodes, s->n_heads, s->head_dim,
                      s->d_state, s->n_groups, max_leaves, max_len};
    hipError_t e = tsv::launch_unroll_gather(u, s->in_dtype == TSV_BF16, (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_ssd_seq_scan(const tsv_shape* s, const void* x_u, const void* dt_u, const float* A,
                             const void* B_u, const void* C_u, const float* D, float* h_inout,
                             const int32_t* seq_len, void* y_u, void* stream) {
    tsv_status st = check_shape(s);
    if (st != TSV_OK) return st;
    if (s->batch == 0 || s->n_nodes == 0) return TSV_OK;
    if (s->head_dim > kBaseMaxDim || s->d_state > kBaseMaxDim ||
        s->head_dim * s->d_state > kBaseMaxState)
        return TSV_E_UNSUPPORTED;
    if ((long long)s->batch * s->n_heads > 0x7fffffffLL) return TSV_E_UNSUPPORTED;
    if (!x_u || !dt_u || !A || !B_u || !C_u || !D || !h_inout || !seq_len || !y_u) return TSV_E_NULL;
    tsv::SeqScanArgs a{x_u, dt_u, A, B_u, C_u, D, h_inout, seq_len, y_u,
                       s->batch, s->n_nodes, s->n_heads, s->head_dim, s->d_state, s->n_groups};
    hipError_t e = tsv::launch_seq_scan(a, s->in_dtype == TSV_BF16, (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_ssd_snapshot_verify(const tsv_shape* s, const void* x, const void* dt, const float* A,
                                    const void* B, const void* C, const float* D, const float* h0,
                                    const int32_t* parent, void* y, float* states, int32_t* tree_status,
                                    void* stream) {
    tsv_status st = check_shape(s);
    if (st != TSV_OK) return st;
    if (s->batch == 0 || s->n_nodes == 0) return TSV_OK;
    if (s->head_dim > kBaseMaxDim || s->d_state > kBaseMaxDim ||
        s->head_dim * s->d_state > kBaseMaxState)
        return TSV_E_UNSUPPORTED;
    if (!x || !dt || !A || !B || !C || !D || !h0 || !parent || !y || !states) return TSV_E_NULL;
    tsv::VerifyArgs a{x,  dt, A,           B,        C,          D,          h0,
                      parent, y, tree_status, s->batch, s->n_nodes, s->n_heads, s->head_dim,
                      s->d_state, s->n_groups};
    hipError_t e = tsv::launch_snapshot_verify(a, states, s->in_dtype == TSV_BF16, (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

tsv_status tree_ssd_snapshot_commit(const tsv_shape* s, const float* states, float* h0_inout,
                                    const int32_t* parent, const int32_t* accepted,
                                    const int32_t* accepted_len, int32_t max_path_len, int32_t* tree_status,
                                    void* stream) {
    tsv_status st = check_shape(s);
    if (st != TSV_OK) return st;
    if (max_path_len < 0 || max_path_len > kMaxNodes) return TSV_E_SHAPE;
    if (s->batch == 0 || s->n_nodes == 0) return TSV_OK;
    if (!states || !h0_inout || !parent || !accepted_len) return TSV_E_NULL;
    if (max_path_len > 0 && !accepted) return TSV_E_NULL;
    hipError_t e = tsv::launch_snapshot_commit(s->batch, s->n_nodes, s->n_heads, s->head_dim * s->d_state,
                                               states, h0_inout, parent, accepted, accepted_len,
                                               max_path_len, tree_status, (hipStream_t)stream);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}

const char* tree_ssd_status_string(int32_t status) {
    switch (status) {
        case TSV_OK: return "ok";
        case TSV_E_NULL: return "null pointer argument";
        case TSV_E_SHAPE: return "size out of range (T > 1024, H % G != 0, negative size, bad heads_per_block or max_path_len)";
        case TSV_E_DTYPE: return "unknown input dtype";
        case TSV_E_UNSUPPORTED: return "unsupported size combination (head_dim or d_state > 256)";
        case TSV_E_LAUNCH: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

int32_t tree_ssd_abi_version(void) { return TREE_SSD_ABI_VERSION; }

}  // extern "C"
