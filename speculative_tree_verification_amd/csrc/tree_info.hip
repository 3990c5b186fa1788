// tree_info.hip -- the tree mask of a packed draft tree: depth and ancestor-or-
// self bit set of every node ("STree: Speculative Tree Decoding for Hybrid
// State Space Models", atlas.scime.ai summary, section "Approach": the mask L
// in A_tree = L log A). One work-group per batch item, one node per thread;
// ancestor sets are built by pointer jumping in LDS (ceil(log2 T) rounds).
// A node's set is max(4, ceil(T / 64)) words: up to 256 nodes 256 threads and
// 4 words, up to 1024 nodes 1024 threads and 16 words (128 KiB of LDS).
#include "common.hpp"
#include "launch.hpp"

namespace tsv {

template <int NT, int W>
__global__ __launch_bounds__(NT) void tree_info_kernel(const int32_t* __restrict__ parent, int T,
                                                      int Wout, int32_t* __restrict__ depth,
                                                      uint64_t* __restrict__ anc,
                                                      int32_t* __restrict__ tree_status) {
    __shared__ int s_par[NT];
    __shared__ int s_nxt[NT];
    __shared__ int s_dep[NT];
    __shared__ uint64_t s_anc[NT][W];

    const int b = blockIdx.x;
    const int i = threadIdx.x;
    const int st = load_tree(parent + (size_t)b * T, T, s_par);
    if (i == 0 && tree_status) tree_status[b] = st;
    if (st) return;

    int nxt = -1, dep = 0;
    uint64_t m[W];
#pragma unroll
    for (int w = 0; w < W; ++w) m[w] = 0;
    if (i < T) {
        nxt = s_par[i];
        dep = (nxt >= 0) ? 1 : 0;
#pragma unroll
        for (int w = 0; w < W; ++w) m[w] = w == (i >> 6) ? (uint64_t)1 << (i & 63) : 0;
        s_nxt[i] = nxt;
        s_dep[i] = dep;
#pragma unroll
        for (int w = 0; w < W; ++w) s_anc[i][w] = m[w];
    }
    // invariant: m = nodes on the path from i up to, but excluding, nxt;
    // dep = number of edges from i to nxt (to the root once nxt < 0)
    while (__syncthreads_or(nxt >= 0)) {
        int n2 = nxt, d2 = dep;
        uint64_t m2[W];
#pragma unroll
        for (int w = 0; w < W; ++w) m2[w] = m[w];
        if (nxt >= 0) {
            d2 = dep + s_dep[nxt];
            n2 = s_nxt[nxt];
#pragma unroll
            for (int w = 0; w < W; ++w) m2[w] |= s_anc[nxt][w];
        }
        __syncthreads();
        if (i < T) {
            s_dep[i] = d2;
            s_nxt[i] = n2;
#pragma unroll
            for (int w = 0; w < W; ++w) s_anc[i][w] = m2[w];
        }
        nxt = n2;
        dep = d2;
#pragma unroll
        for (int w = 0; w < W; ++w) m[w] = m2[w];
    }
    if (i < T) {
        depth[(size_t)b * T + i] = dep;
        uint64_t* o = anc + ((size_t)b * T + i) * Wout;
#pragma unroll
        for (int w = 0; w < W; ++w)
            if (w < Wout) o[w] = m[w];
    }
}

hipError_t launch_tree_info(int batch, int T, const int32_t* parent, int32_t* depth,
                            uint64_t* anc, int32_t* tree_status, hipStream_t stream) {
    const int Wout = anc_words(T);
    if (T <= kMaxNodes)
        hipLaunchKernelGGL((tree_info_kernel<kMaxNodes, 4>), dim3(batch), dim3(kMaxNodes), 0,
                           stream, parent, T, Wout, depth, anc, tree_status);
    else
        hipLaunchKernelGGL((tree_info_kernel<kMaxNodesLarge, kMaxNodesLarge / 64>), dim3(batch),
                           dim3(kMaxNodesLarge), 0, stream, parent, T, Wout, depth, anc,
                           tree_status);
    return hipGetLastError();
}

}  // namespace tsv
