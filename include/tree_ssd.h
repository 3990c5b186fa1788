/*
 * tree_ssd.h -- C ABI of libtree_ssd.so: packed-tree verification and commit
 * for one Mamba2/SSD layer on AMD MI355X (gfx950).
 *
 * Method: "STree: Speculative Tree Decoding for Hybrid State Space Models"
 * (atlas.scime.ai summary, sections "Problem" and "Approach"; mlsanity
 * abstract). A draft token tree is packed into one sequence of T nodes, node 0
 * the root and every parent listed before its children. One pass gives every
 * node the exact output the SSM recurrence would give on that node's root path
 * alone. The tree mask L (ancestor-or-self) accumulates the per-token log
 * decays along root paths ("A_tree = L log A", read with log A_j = dt_j * A_h,
 * the log of the discrete transition exp(dt_j * A_h)). Commit ("activation
 * replay for state backtracking") rebuilds only the accepted path's final
 * state from the retained inputs; no per-node state is ever stored.
 *
 * Per batch item b and head h (group g = h / (H / G)), with the state stored
 * as H[p][n] (P x N, n fastest):
 *   H_i = exp(cum_i) h0 + sum_{j on path(i)} exp(cum_i - cum_j) dt_j x_j (outer) B_j
 *   y_i = H_i C_i + D_h x_i,      cum_i = sum_{j on path(i)} dt_j A_h
 * which is the recurrence H <- exp(dt A) H + dt x (outer) B, y = H C + D x run
 * from h0 along the root path of node i.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *     row-major. The library allocates nothing, keeps no state between calls,
 *     and is reentrant, with one exception: tree_ssd_commit_layers_static
 *     keeps its layer table in a fixed device array of the library's (one per
 *     GPU), so its calls that overlap on one GPU race. Work is enqueued on
 *     `stream` (a hipStream_t; NULL means
 *     the null stream) without synchronising; results are ready when the
 *     stream reaches that point.
 *   - Host-detectable errors (NULL pointers, bad sizes, bad dtype) return a
 *     tsv_status other than TSV_OK before anything is enqueued.
 *   - Data-dependent errors are reported per batch item in device memory
 *     tree_status[b] (a bit set, see TSV_ST_*). The outputs of an item with any
 *     bit set are left bitwise untouched. tree_status may be NULL (no report;
 *     invalid items are still skipped).
 *   - Nodes are limited to T <= 1024. bf16 inputs with head_dim 64 and
 *     d_state 64 or 128 take MFMA verify kernels at every tree size; other
 *     shapes and fp32 inputs take plain fp32 kernels (same results, lower
 *     throughput).
 *   - The launch runs on the device current to the calling thread.
 */
#ifndef TREE_SSD_H
#define TREE_SSD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of x, dt, B, C and y */
typedef enum { TSV_F32 = 0, TSV_BF16 = 1 } tsv_dtype;

/* Return codes */
typedef enum {
    TSV_OK = 0,
    TSV_E_NULL = 1,        /* a required pointer is NULL */
    TSV_E_SHAPE = 2,       /* a size is out of range, H % G != 0, or T > 1024 */
    TSV_E_DTYPE = 3,       /* in_dtype is not a tsv_dtype */
    TSV_E_UNSUPPORTED = 4, /* the size combination has no kernel (this includes
                              head_dim or d_state above 256 and more than
                              65535 heads) */
    TSV_E_LAUNCH = 5       /* the HIP launch failed (see hipGetLastError) */
} tsv_status;

/* Per-item status bits written to tree_status[b] */
#define TSV_ST_BAD_ROOT 1   /* parent[b][0] != -1 */
#define TSV_ST_BAD_PARENT 2 /* some parent[b][i] (i >= 1) is not in [0, i) */
#define TSV_ST_BAD_PATH 4   /* accepted path: len not in [0, max_path_len]
                               or above T, first node not 0, an index not in
                               [0, T), or a node whose parent is not the
                               previous entry */

/* Flags (tsv_shape.flags) */
#define TSV_FLAG_FORCE_GENERIC 1 /* use the plain VALU verify kernel even where
                                    the MFMA kernel applies (testing aid) */
#define TSV_FLAG_FORCE_WIDE 2    /* use the wide-tree MFMA verify kernel for any
                                    tree size it supports (testing / tuning aid) */
#define TSV_FLAG_FORCE_SMALL 4   /* trees of at most 16 nodes: use the 64-node
                                    small-tree MFMA kernel instead of the one-wave
                                    tiny-tree kernel (testing / tuning aid) */

typedef struct {
    int32_t batch;           /* Bt >= 0 (0: nothing to do) */
    int32_t n_nodes;         /* T in [0, 1024] (0: nothing to do) */
    int32_t n_heads;         /* H >= 1 */
    int32_t head_dim;        /* P >= 1 */
    int32_t d_state;         /* N >= 1 */
    int32_t n_groups;        /* G >= 1, H % G == 0; head h uses group h / (H/G) */
    int32_t in_dtype;        /* tsv_dtype of x, dt, B, C, y */
    int32_t flags;           /* TSV_FLAG_* (0 = automatic choice) */
    int32_t heads_per_block; /* launch hint: heads one work-group handles for the
                                MFMA verify kernel; 0 = automatic. Must divide
                                H / G when given. The tiny-tree kernel
                                (T <= 16) takes one head_dim slice per
                                work-group and ignores it. */
} tsv_shape;

/*
 * tree_ssd_verify -- every node's output of one SSD layer over a packed tree
 * (the summary's section "Approach": log decays summed along ancestor paths let
 * one pass over the packed tree give each node the output of its own root path,
 * exactly).
 *
 *   x      [Bt][T][H][P]   in_dtype   token inputs
 *   dt     [Bt][T][H]      in_dtype   step sizes, already positive (after any
 *                                     softplus / bias of the caller)
 *   A      [H]             float      per-head decay rate (normally < 0)
 *   B, C   [Bt][T][G][N]   in_dtype   input / output projections
 *   D      [H]             float      skip weight
 *   h0     [Bt][H][P][N]   float      state before the root (read only)
 *   parent [Bt][T]         int32      parent[b][0] = -1, parent[b][i] in [0, i)
 *   y      [Bt][T][H][P]   in_dtype   output (bf16 results rounded to nearest
 *                                     even from fp32 accumulators)
 *   tree_status [Bt]       int32      optional; set to bits 1|2 of the item's tree
 *
 * Arithmetic: fp32 accumulation throughout. For bf16 inputs with P == 64 and
 * N in {64, 128} the h0 read-out C h0^T runs on bf16 MFMA with h0 split into a
 * bf16 high and low part (about 16 significant bits). For trees of more than
 * 64 nodes the masked decay weights of the intra-tree term are rounded once to
 * bf16 for the bf16 dot-product instruction, except the node's own weight
 * (which carries D) and its parent's, which keep about 16 bits. Other inputs
 * and shapes use fp32 arithmetic on the (exact) input values.
 */
tsv_status tree_ssd_verify(const tsv_shape* s, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, const float* h0,
                           const int32_t* parent, void* y, int32_t* tree_status, void* stream);

/*
 * tree_ssd_commit -- overwrite h0 with the state at the end of the accepted
 * root path by replaying the path's tokens (the summary's section "Approach":
 * state is restored from the retained activations rather than from per-node
 * snapshots), using the same inputs the verify call read:
 *   H' = exp(cum_l) h0 + sum_k exp(cum_l - cum_{j_k}) dt_{j_k} x_{j_k} (outer) B_{j_k}
 * for the path j_0 = 0, ..., j_{len-1} = l. len == 0 leaves h0 unchanged.
 *
 *   x, dt, A, B, parent   as for tree_ssd_verify (only path rows are read)
 *   h0_inout [Bt][H][P][N] float   read, then overwritten in place
 *   accepted [Bt][max_path_len] int32  root-path node list of each item
 *   accepted_len [Bt]      int32   number of valid entries of each row
 *   max_path_len           >= 0    row length of `accepted` (1 <= ... <= 1024
 *                                  when Bt > 0; 0 allowed with all len == 0)
 *   tree_status [Bt]       int32   optional; bits 1|2|4 of the item
 *
 * Not idempotent: a second call advances the state again. It must be ordered
 * after every verify that reads the same h0 (same stream, or an event).
 */
tsv_status tree_ssd_commit(const tsv_shape* s, const void* x, const void* dt, const float* A,
                           const void* B, float* h0_inout, const int32_t* parent,
                           const int32_t* accepted, const int32_t* accepted_len,
                           int32_t max_path_len, int32_t* tree_status, void* stream);

/* One layer's operands for tree_ssd_commit_layers: device pointers with the
 * layouts of tree_ssd_commit (x, dt, B in in_dtype; A float; h0 float). */
typedef struct {
    const void* x;   /* [Bt][T][H][P] */
    const void* dt;  /* [Bt][T][H]    */
    const float* A;  /* [H]           */
    const void* B;   /* [Bt][T][G][N] */
    float* h0_inout; /* [Bt][H][P][N] read, then overwritten in place */
} tsv_commit_layer;

/*
 * tree_ssd_commit_layers -- tree_ssd_commit for n_layers layers of one model
 * step in a single launch. All layers share the shape, the draft tree and the
 * accepted path: one decoding step accepts the same tokens in every layer
 * (the summary's section "Approach": every layer's state is rebuilt from its
 * own retained inputs along that path). Once the path is known the layers are
 * independent, so their commits need not run one after another; each layer's
 * result is exactly that of tree_ssd_commit on its operands.
 *
 *   n_layers    >= 0    number of entries of `layers` (0: nothing to do)
 *   layers      device array [n_layers] of tsv_commit_layer, owned by the
 *               caller, read by the kernel (so it must stay valid until the
 *               stream passes this call); no two entries may share h0_inout
 *   parent, accepted, accepted_len, max_path_len
 *               as for tree_ssd_commit, shared by all layers
 *   tree_status [Bt]    optional; written once per item (bits 1|2|4)
 *
 * An item whose tree or path is invalid keeps h0 untouched in every layer.
 * Returns TSV_E_NULL for a NULL `layers` with n_layers > 0 and TSV_E_SHAPE for
 * n_layers < 0; the pointers inside the table are not checked on the host.
 */
tsv_status tree_ssd_commit_layers(const tsv_shape* s, int32_t n_layers,
                                  const tsv_commit_layer* layers, const int32_t* parent,
                                  const int32_t* accepted, const int32_t* accepted_len,
                                  int32_t max_path_len, int32_t* tree_status, void* stream);

/* Most layers tree_ssd_commit_layers_static takes in one call. */
#define TSV_STATIC_MAX_LAYERS 1024

/*
 * tree_ssd_commit_layers_static -- tree_ssd_commit_layers for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * that must not call hipMalloc, harnesses that forbid it. The layer table is
 * passed in HOST memory; the call stages it into a fixed device array that
 * the library holds for the life of the process (TSV_STATIC_MAX_LAYERS
 * entries of 40 bytes, one copy per GPU, its address looked up on the first
 * call made on that GPU) and then runs the commit kernel of
 * tree_ssd_commit_layers on it, so the results are bitwise those of that
 * call. Nothing is allocated or freed.
 *
 *   layers_host  host array [n_layers] of tsv_commit_layer (device pointers
 *                inside, as for tree_ssd_commit_layers); read during the
 *                call, which passes it to the GPU as kernel arguments (64
 *                entries per staging launch), so it may be freed or reused as
 *                soon as the call returns
 *   every other argument as for tree_ssd_commit_layers.
 *
 * Returns TSV_E_UNSUPPORTED for n_layers > TSV_STATIC_MAX_LAYERS, TSV_E_NULL
 * for a NULL layers_host with n_layers > 0, TSV_E_LAUNCH if the device array
 * cannot be resolved, and otherwise what tree_ssd_commit_layers returns.
 * Every call on one GPU shares that GPU's array and overwrites the entries it
 * uses: two calls whose work overlaps on one GPU (different streams, no
 * ordering between them) race. Calls ordered on one stream do not.
 */
tsv_status tree_ssd_commit_layers_static(const tsv_shape* s, int32_t n_layers,
                                         const tsv_commit_layer* layers_host, const int32_t* parent,
                                         const int32_t* accepted, const int32_t* accepted_len,
                                         int32_t max_path_len, int32_t* tree_status, void* stream);

/*
 * tree_gdn_verify -- every node's output of one gated-delta-rule layer over a
 * packed tree ("TreeWY: Speculative Verification for Gated DeltaNet Hybrids",
 * fugumt page, abstract: one triangular solve over the tree gives every draft
 * node's output, and a small pseudo-value matrix is kept for commit). Per head
 * the state S (dv x dk, stored [p][n]) follows
 *   S <- exp(g) S (I - beta k k^T) + beta v k^T,   o = S q
 * from S0 along each node's root path. With G_i the sum of g over that path,
 * the pseudo-values e solve
 *   e_i + beta_i sum_{j strict ancestor of i} exp(G_i - G_j) (k_i . k_j) e_j
 *       = beta_i (v_i - exp(G_i) S0 k_i)
 * and o_i = exp(G_i) S0 q_i + sum_{j on path(i)} exp(G_i - G_j) (q_i . k_j) e_j.
 *
 * The shape uses tsv_shape with head_dim = dv, d_state = dk, n_groups = 1;
 * in_dtype is the type of q, k, v and o: TSV_F32 or TSV_BF16 (bf16 bit
 * patterns); g, beta, S0 and e are fp32 either way. n_nodes <= 256, dk and
 * dv <= 128 (TSV_E_UNSUPPORTED otherwise). Trees of 65 to 256 nodes take a
 * second kernel, which holds the tree's pair tables in LDS: a tree with more
 * than 4096 ancestor-or-self pairs (the sum over nodes of depth + 1) sets
 * status bit 8 and is left untouched.
 *   q, k   [Bt][T][H][dk]   queries and keys (keys normally of unit length)
 *   v      [Bt][T][H][dv]   values
 *   g      [Bt][T][H]       log gate (<= 0)
 *   beta   [Bt][T][H]       step in [0, 1]
 *   S0     [Bt][H][dv][dk]  state before the root (read only)
 *   parent [Bt][T]          as for tree_ssd_verify
 *   o      [Bt][T][H][dv]   output (in_dtype; bf16 rounded to nearest even)
 *   e      [Bt][T][H][dv]   optional output, fp32: the pseudo-values, input of commit
 *   tree_status [Bt]        optional; bits 1|2, and 8 as above
 * fp32 arithmetic throughout (bf16 inputs are exact in it).
 */
tsv_status tree_gdn_verify(const tsv_shape* s, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const float* S0,
                           const int32_t* parent, void* o, float* e, int32_t* tree_status,
                           void* stream);

/*
 * tree_gdn_commit -- overwrite S0 with the state at the end of each item's
 * accepted root path from the pseudo-values tree_gdn_verify wrote:
 *   S' = exp(G_l) S0 + sum_{j on the path} exp(G_l - G_j) e_j k_j^T.
 * k (in_dtype), g, parent as for tree_gdn_verify; e (fp32) from it; accepted, accepted_len,
 * max_path_len and tree_status (bits 1|2|4) as for tree_ssd_commit. len == 0
 * leaves S0 unchanged; invalid items leave it untouched. Past 64 nodes,
 * max_path_len must be at most 128 (TSV_E_UNSUPPORTED otherwise): the path's
 * rows are staged whole in LDS.
 */
tsv_status tree_gdn_commit(const tsv_shape* s, const void* k, const float* g, const float* e,
                           float* S0_inout, const int32_t* parent, const int32_t* accepted,
                           const int32_t* accepted_len, int32_t max_path_len, int32_t* tree_status,
                           void* stream);

/*
 * tree_ssd_accept_greedy -- the accepted root path of each verified tree at
 * temperature 0, the input of tree_ssd_commit. The target model's choice
 * after node i is target_tokens[i] (its argmax next token); a child c of an
 * accepted node i is accepted when draft_tokens[c] == target_tokens[i]
 * ("TreeSpark: Adaptive Draft Trees Accelerate Speculative Decoding by
 * 8-14%", section on the lossless guarantee: the target model keeps or rejects
 * draft tokens, and a draft tree offers several candidate paths checked in one
 * pass). The root (node 0, the token the tree grows from) is always accepted.
 * The path is the deepest root path whose every non-root node is accepted; a
 * tree without repeated sibling tokens has at most one, and with repeats the
 * deepest accepted node of smallest index ends the path.
 *
 *   parent        [Bt][T] int32   as for tree_ssd_verify
 *   draft_tokens  [Bt][T] int32   token of each node (node 0: the root token)
 *   target_tokens [Bt][T] int32   target model's greedy next token after each node
 *   max_path_len  in [1, 1024]    row length of `accepted`
 *   accepted      [Bt][max_path_len] int32  output: node indices of the path,
 *                                 root first, cut after max_path_len entries;
 *                                 entries past the length are -1
 *   accepted_len  [Bt] int32      output: entries of the path kept (>= 1)
 *   next_token    [Bt] int32      optional output: target token after the last
 *                                 kept node (the token the next step starts from)
 *   tree_status   [Bt] int32      optional; bits 1|2 of the item's tree
 * Invalid items leave accepted, accepted_len and next_token untouched.
 */
tsv_status tree_ssd_accept_greedy(int32_t batch, int32_t n_nodes, const int32_t* parent,
                                  const int32_t* draft_tokens, const int32_t* target_tokens,
                                  int32_t max_path_len, int32_t* accepted, int32_t* accepted_len,
                                  int32_t* next_token, int32_t* tree_status, void* stream);

#define TSV_ST_BAD_TOKEN 16 /* a non-root draft token is outside [0, vocab) */

/*
 * tree_ssd_accept_stochastic -- the accepted root path of each verified tree
 * at temperature > 0: multi-step speculative sampling over the tree with
 * siblings drawn without replacement ("STree: Speculative Tree Decoding for
 * Hybrid State-Space Models", atlas.scime.ai summary, measured-effects table:
 * multi-step speculative sampling; "TreeSpark: Adaptive Draft Trees
 * Accelerate Speculative Decoding by 8-14%", section on the lossless
 * guarantee: siblings sampled without replacement and rejected tokens
 * resampled from the residual, recursively). The produced tokens follow the
 * target's distribution whatever the draft's.
 *
 * Starting at the root with residual r = p_target[root], the children of the
 * current node u are tested in increasing index. The k-th child's token t was
 * drawn from d = q_draft[u] without the earlier children's tokens, divided by
 * m = 1 - (their draft mass) (d = 0 when m <= 0 or t repeats an earlier
 * sibling's token). It is accepted when u_node[c] * d[t] < r[t]; an accepted
 * child becomes u. A rejection replaces r by max(r - d, 0) divided by its mass
 * (r is kept when that mass is 0). When no child is accepted, next_token is
 * the first token whose running sum of r exceeds u_final times r's total
 * (-1 if r has no mass). The path is cut after max_path_len nodes; a child
 * accepted below the cut gives next_token instead (its token is a draw from
 * the cut node's target). Decisions are taken in fp64; sums over the
 * vocabulary are taken in an order of the kernel's own, so a decision can
 * differ from a left-to-right evaluation only within fp64 rounding of its
 * threshold.
 *
 *   n_nodes       in [1, 1024]; vocab >= 1
 *   parent        [Bt][T] int32   as for tree_ssd_verify
 *   draft_tokens  [Bt][T] int32   token of each node (node 0's is not used)
 *   p_target      [Bt][T][vocab] float32  target distribution of the token
 *                                 after each node (rows sum to 1)
 *   q_draft       [Bt][T][vocab] float32  draft distribution the children of
 *                                 each node drew their tokens from, one after
 *                                 another without replacement, in index order
 *   u_node        [Bt][T] float32 uniforms in [0, 1): each non-root node's test
 *   u_final       [Bt] float32    uniform in [0, 1) of each item's final draw
 *   max_path_len  in [1, 1024]    row length of `accepted`
 *   accepted      [Bt][max_path_len] int32  output: node indices of the path,
 *                                 root first; entries past the length are -1
 *   accepted_len  [Bt] int32      output: entries of the path (>= 1)
 *   next_token    [Bt] int32      optional output: the token after the path
 *   tree_status   [Bt] int32      optional; bits 1|2 of the item's tree, and
 *                                 TSV_ST_BAD_TOKEN
 * Only the rows of visited nodes are read (one pass over p_target and q_draft
 * of a node per rejected child, one more for the final draw). No workspace:
 * the residual is never stored. Invalid items leave accepted, accepted_len and
 * next_token untouched. Returns TSV_E_SHAPE for sizes out of range and
 * TSV_E_NULL for a NULL required pointer.
 */
tsv_status tree_ssd_accept_stochastic(int32_t batch, int32_t n_nodes, int32_t vocab,
                                      const int32_t* parent, const int32_t* draft_tokens,
                                      const float* p_target, const float* q_draft, const float* u_node,
                                      const float* u_final, int32_t max_path_len, int32_t* accepted,
                                      int32_t* accepted_len, int32_t* next_token, int32_t* tree_status,
                                      void* stream);

/*
 * tree_ssd_tree_info -- the tree mask of each item (the summary's L): depth of
 * every node (edges from the root) and its ancestor-or-self set as W 64-bit
 * words, W = max(4, ceil(n_nodes / 64)) (bit j % 64 of word j / 64 set iff
 * node j is on the root path of node i); four words up to 256 nodes.
 *
 *   parent   [batch][n_nodes] int32
 *   depth    [batch][n_nodes] int32     output
 *   anc_bits [batch][n_nodes][W] uint64 output (unused words are zero)
 *   tree_status [batch] int32           optional; bits 1|2
 * Invalid items leave depth and anc_bits untouched.
 */
tsv_status tree_ssd_tree_info(int32_t batch, int32_t n_nodes, const int32_t* parent,
                              int32_t* depth, uint64_t* anc_bits, int32_t* tree_status,
                              void* stream);

/* ------------------------------------------------------------------------
 * The two forms a packed tree replaces, on the same inputs, for measuring it
 * against them ("STree: Speculative Tree Decoding for Hybrid State Space
 * Models", atlas.scime.ai summary: without a packed-tree scan an SSM unrolls
 * the draft tree into repeated sequences with extra states and memory, section
 * "Problem"; the paper's baseline is a fused selective scan over the unrolled
 * tree, section "Experimental setup", times in "Key results". The Bole and
 * TreeWY abstracts, mlsanity and fugumt pages, describe the other form: a full
 * recurrent state materialised for every draft node).
 * ------------------------------------------------------------------------ */

/* Per-item status bit of tree_ssd_unroll_plan: more leaves than max_leaves, or
 * a root path longer than max_len */
#define TSV_ST_OVER_CAPACITY 8

/*
 * tree_ssd_unroll_plan -- the unrolled form of each item's tree: one sequence
 * per leaf (a node that is no node's parent, leaves taken by increasing
 * index), holding the leaf's root path from node 0.
 *
 *   parent     [Bt][T] int32
 *   max_leaves in [1, 1024]   sequence slots per item (Lcap)
 *   max_len    in [1, 1024]   positions per sequence (S)
 *   seq_nodes  [Bt][Lcap][S] int32  output: node at each position, -1 past the end
 *   seq_len    [Bt][Lcap] int32     output: path length, 0 for unused slots
 *   n_leaves   [Bt] int32           output: sequences of the item
 *   tree_status [Bt] int32          optional; bits 1|2, or TSV_ST_OVER_CAPACITY
 * Every output is written for every item: an invalid or over-capacity item
 * gets n_leaves 0 and empty slots.
 */
tsv_status tree_ssd_unroll_plan(int32_t batch, int32_t n_nodes, const int32_t* parent, int32_t max_leaves,
                                int32_t max_len, int32_t* seq_nodes, int32_t* seq_len, int32_t* n_leaves,
                                int32_t* tree_status, void* stream);

/*
 * tree_ssd_unroll_gather -- materialise the unrolled sequences: for sequence
 * q = b * max_leaves + l and position s < seq_len[q], copy node
 * n = seq_nodes[q][s]'s rows, and give every sequence its own copy of h0[b].
 * Layouts follow the packed ones with (item, leaf) as the batch index:
 *   x_u [Bt*Lcap][S][H][P], dt_u [Bt*Lcap][S][H], B_u, C_u [Bt*Lcap][S][G][N]
 *   (in_dtype), h0_u [Bt*Lcap][H][P][N] float.
 * s gives the packed shape (x, dt, B, C, h0 as for tree_ssd_verify). Positions
 * past a sequence's length and sequences of length 0 are not written; a
 * length outside [0, S] or a node index outside [0, T) skips the slot.
 */
tsv_status tree_ssd_unroll_gather(const tsv_shape* s, int32_t max_leaves, int32_t max_len, const void* x,
                                  const void* dt, const void* B, const void* C, const float* h0,
                                  const int32_t* seq_nodes, const int32_t* seq_len, void* x_u, void* dt_u,
                                  void* B_u, void* C_u, float* h0_u, void* stream);

/*
 * tree_ssd_seq_scan -- an ordinary Mamba2 scan over sequences (no tree): for
 * each sequence q and head h, from the state h_inout[q][h],
 *   H <- exp(dt_t A_h) H + dt_t x_t (outer) B_t,   y_t = H C_t + D_h x_t
 * for t < seq_len[q]; the final state is written back to h_inout. The shape's
 * batch is the number of sequences and n_nodes their row count S; layouts as
 * written by tree_ssd_unroll_gather, y_u like x_u. head_dim, d_state <= 256
 * and head_dim * d_state <= 16384 (TSV_E_UNSUPPORTED otherwise). Sequences
 * whose length is outside [1, S] are skipped. fp32 arithmetic.
 */
tsv_status tree_ssd_seq_scan(const tsv_shape* s, const void* x_u, const void* dt_u, const float* A,
                             const void* B_u, const void* C_u, const float* D, float* h_inout,
                             const int32_t* seq_len, void* y_u, void* stream);

/*
 * tree_ssd_snapshot_verify -- every node's state materialised: states[b][h][i]
 * is the state after node i's root path (formed from the parent's stored
 * state), and y_i = states_i C_i + D x_i. Arguments as for tree_ssd_verify,
 * plus
 *   states [Bt][H][T][P][N] float  output (T * P * N * 4 bytes per item and head)
 * head_dim, d_state <= 256, head_dim * d_state <= 16384. An invalid item
 * leaves y and states untouched. fp32 arithmetic.
 */
tsv_status tree_ssd_snapshot_verify(const tsv_shape* s, const void* x, const void* dt, const float* A,
                                    const void* B, const void* C, const float* D, const float* h0,
                                    const int32_t* parent, void* y, float* states, int32_t* tree_status,
                                    void* stream);

/*
 * tree_ssd_snapshot_commit -- the snapshot form's commit: copy the stored state
 * of each item's last accepted node into h0_inout [Bt][H][P][N]. states as
 * written by tree_ssd_snapshot_verify; parent, accepted, accepted_len,
 * max_path_len and tree_status (bits 1|2|4) as for tree_ssd_commit. len == 0
 * leaves h0 unchanged; an invalid item leaves it untouched.
 */
tsv_status tree_ssd_snapshot_commit(const tsv_shape* s, const float* states, float* h0_inout,
                                    const int32_t* parent, const int32_t* accepted,
                                    const int32_t* accepted_len, int32_t max_path_len, int32_t* tree_status,
                                    void* stream);

/* Static, human-readable name of a tsv_status value. */
const char* tree_ssd_status_string(int32_t status);

/* ABI version of this header (incremented on any incompatible change). */
int32_t tree_ssd_abi_version(void);

#define TREE_SSD_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* TREE_SSD_H */
