// accept.hip -- greedy acceptance of a verified draft tree: the step between
// verify and commit. At temperature 0 the target model's choice after node i
// is its argmax token target[i]; a child c of an accepted node is accepted
// when its draft token equals that choice ("TreeSpark: Adaptive Draft Trees
// Accelerate Speculative Decoding by 8-14%", section on the lossless
// guarantee: draft tokens are kept or rejected by the target model, and a
// draft tree offers several candidate paths checked in one pass; "STree:
// Speculative Tree Decoding for Hybrid State-Space Models", mlsanity summary,
// key facts: runs at temperature 0). The root is the token the tree grows
// from and is always accepted. The accepted path is the deepest root path
// whose every non-root node matches; without repeated sibling tokens at most
// one path matches, with repeats the deepest matching node of smallest index
// is taken.
//
// One work-group per item, one thread per node (256 threads, or 1024 for trees
// past 256 nodes). After validation every node
// tests its own match against its parent's target token; pointer jumping over
// the tree (log2 depth rounds in LDS) gives each node its depth and whether
// its whole root path matches; an LDS max over (depth, -index) picks the last
// accepted node, whose root path is then written root first.
#include "common.hpp"
#include "launch.hpp"

namespace tsv {

template <int NT>
__global__ __launch_bounds__(NT) void accept_greedy_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ target, int T, int Lmax, int32_t* __restrict__ accepted,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ next_token,
    int32_t* __restrict__ tree_status) {
    __shared__ int s_par[NT];
    __shared__ int s_tgt[NT];
    __shared__ int s_nxt[NT];
    __shared__ int s_dep[NT];
    __shared__ int s_ok[NT];
    __shared__ int s_path[NT];
    __shared__ int s_best;
    const int b = blockIdx.x;
    const int i = threadIdx.x;
    const int p = load_parent(parent + (size_t)b * T, T);
    const int ic = min(i, T - 1);
    const int tok = draft[(size_t)b * T + ic];
    const int tgt = target[(size_t)b * T + ic];
    const int st = check_tree(p, T, s_par);
    if (i == 0 && tree_status) tree_status[b] = st;
    if (st) return;
    if (i < T) s_tgt[i] = tgt;
    if (i == 0) s_best = -1;
    __syncthreads();
    // own match, then AND and depth accumulated along the root path
    int nxt = i < T ? p : -1;
    int dep = nxt >= 0 ? 1 : 0;
    int ok = i < T && (i == 0 || tok == s_tgt[p]);
    if (i < T) {
        s_nxt[i] = nxt;
        s_dep[i] = dep;
        s_ok[i] = ok;
    }
    while (__syncthreads_or(nxt >= 0)) {
        int n2 = nxt, d2 = dep, o2 = ok;
        if (nxt >= 0) {
            d2 = dep + s_dep[nxt];
            o2 = ok & s_ok[nxt];
            n2 = s_nxt[nxt];
        }
        __syncthreads();
        if (i < T) {
            s_dep[i] = d2;
            s_ok[i] = o2;
            s_nxt[i] = n2;
        }
        nxt = n2;
        dep = d2;
        ok = o2;
    }
    // deepest fully matching node, smallest index among equals: key (depth,
    // 1023 - index), 10 bits of index
    if (ok) atomicMax(&s_best, (dep << 10) | (1023 - i));
    __syncthreads();
    const int best = s_best;  // the root always matches, so best >= 0
    const int last = 1023 - (best & 1023);
    const int dl = best >> 10;
    if (i == 0) {
        int j = last;
        for (int k = dl; k >= 0; --k) {
            s_path[k] = j;
            j = s_par[j];
        }
    }
    __syncthreads();
    const int len = min(dl + 1, Lmax);
    for (int k = i; k < Lmax; k += NT) accepted[(size_t)b * Lmax + k] = k < len ? s_path[k] : -1;
    if (i == 0) {
        accepted_len[b] = len;
        if (next_token) next_token[b] = s_tgt[s_path[len - 1]];
    }
}

hipError_t launch_accept_greedy(int batch, int T, const int32_t* parent, const int32_t* draft,
                                const int32_t* target, int Lmax, int32_t* accepted,
                                int32_t* accepted_len, int32_t* next_token, int32_t* tree_status,
                                hipStream_t stream) {
    if (T <= kMaxNodes)
        hipLaunchKernelGGL(accept_greedy_kernel<kMaxNodes>, dim3(batch), dim3(kMaxNodes), 0, stream,
                           parent, draft, target, T, Lmax, accepted, accepted_len, next_token,
                           tree_status);
    else
        hipLaunchKernelGGL(accept_greedy_kernel<kMaxNodesLarge>, dim3(batch), dim3(kMaxNodesLarge),
                           0, stream, parent, draft, target, T, Lmax, accepted, accepted_len,
                           next_token, tree_status);
    return hipGetLastError();
}

}  // namespace tsv
