// verify_common.hpp -- pieces shared by the two bf16 MFMA verify kernels
// (small trees: verify_mfma.hip; wide trees: verify_wide.hip).
//
// Both compute, per (item b, head h), for every node i of the packed tree
// ("STree: Speculative Tree Decoding for Hybrid State Space Models",
// atlas.scime.ai summary, section "Approach"):
//   y_i = exp(cum_i) (h0 C_i) + sum_{j on path(i)} G_ij exp(cum_i - cum_j) dt_j x_j + D x_i
// with G = C B^T evaluated on ancestor pairs only.
#pragma once

#include "common.hpp"

namespace tsv {

constexpr int kHeadDim = 64;  // head_dim of the MFMA kernels: 4 row tiles of 16

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float s) {
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x),
                                        __builtin_bit_cast(bf16x2, b.x), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y),
                                        __builtin_bit_cast(bf16x2, b.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z),
                                        __builtin_bit_cast(bf16x2, b.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w),
                                        __builtin_bit_cast(bf16x2, b.w), s, false);
    return s;
}

// Dot product of two bf16 rows of N elements (16-byte aligned), all loads
// issued before the first use so one memory round trip covers the row.
template <int N>
__device__ __forceinline__ float dot_rows(const uint16_t* __restrict__ a,
                                          const uint16_t* __restrict__ b) {
    constexpr int V = N / 8;
    uint4 va[V], vb[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        va[v] = *(const uint4*)(a + 8 * v);
        vb[v] = *(const uint4*)(b + 8 * v);
    }
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int v = 0; v < V; v += 2) {
        s0 = dot8_bf16(va[v], vb[v], s0);
        if (v + 1 < V) s1 = dot8_bf16(va[v + 1], vb[v + 1], s1);
    }
    return s0 + s1;
}

// Same dot product with one 16-byte chunk pair in flight at a time (few
// registers; for rarely taken paths).
template <int N>
__device__ __forceinline__ float dot_rows_lean(const uint16_t* __restrict__ a,
                                               const uint16_t* __restrict__ b) {
    float s = 0.f;
#pragma unroll 1
    for (int v = 0; v < N / 8; ++v) s = dot8_bf16(*(const uint4*)(a + 8 * v), *(const uint4*)(b + 8 * v), s);
    return s;
}

// Pair scores with four lanes per pair: lane part (0..3) of a group of four
// consecutive lanes takes a quarter of the row, and the partial sums are
// combined with two cross-lane exchanges. Every group of four lanes handles one
// pair; groups past `count` still take part in the exchanges.
template <int N, typename RowFn>
__device__ __forceinline__ void pair_scores_x4(int count, const uint16_t* s_pair_tab, float* s_out,
                                               RowFn rows) {
    constexpr int V = N / 32;  // 16-byte chunks per quarter row
    const int part = threadIdx.x & 3;
    const int rounds = (4 * count + kBlock - 1) / kBlock;
    for (int rd = 0; rd < rounds; ++rd) {
        const int pq = (rd * kBlock + (int)threadIdx.x) >> 2;
        float s = 0.f;
        if (pq < count) {
            const int pr = s_pair_tab[pq];
            const uint16_t* a;
            const uint16_t* b;
            rows(pr & 255, pr >> 8, a, b);
            uint4 va[V], vb[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                va[v] = *(const uint4*)(a + 8 * (part * V + v));
                vb[v] = *(const uint4*)(b + 8 * (part * V + v));
            }
#pragma unroll
            for (int v = 0; v < V; ++v) s = dot8_bf16(va[v], vb[v], s);
        }
        s += __shfl_xor(s, 1, kWave);
        s += __shfl_xor(s, 2, kWave);
        if (pq < count && part == 0) s_out[pq] = s;
    }
}

// Split 8 fp32 values into bf16 high parts and bf16 residuals (hi + lo carries
// about 16 significant bits of each value).
__device__ __forceinline__ void split_hi_lo(const float4& a, const float4& b, bf16x8& hi,
                                            bf16x8& lo) {
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 hb = (__bf16)f[e];
        hi[e] = hb;
        lo[e] = (__bf16)(f[e] - (float)hb);
    }
}

// Tree set-up shared by the verify kernels, run by all NT threads after the
// tree has been validated: depth (walks to the root for shallow trees, else
// pointer jumping), the ancestor-pair list of
// every node (node i's pairs occupy [s_off[i], s_off[i] + s_dep[i] + 1), from
// i itself up to the root; entry = i | j << 8), and the total pair count.
// Pairs are written only when they fit in max_pairs. s_scratch needs
// kMaxNodes ints and is clobbered.
// All barriers are LDS-only: global loads issued before the call stay in flight.
// s_scan holds at least NT/64 ints.
template <int NT = kBlock>
__device__ __forceinline__ int build_pairs(const int* s_par, int T, int* s_dep, int* s_off,
                                           int* s_scratch, int* s_scan, uint16_t* s_pair,
                                           int max_pairs) {
    const int tid = threadIdx.x;
    const int dep = tree_depth_shallow<NT>(s_par, T, s_scratch, s_dep, s_scan);
    int total;
    const int off = block_exclusive_scan<NT, true>(tid < T ? dep + 1 : 0, s_scan, &total);
    if (tid < T) {
        s_off[tid] = off;
        s_dep[tid] = dep;
        if (total <= max_pairs) {
            int k = 0;
            for (int j = tid; j >= 0; j = s_par[j]) s_pair[off + k++] = (uint16_t)(tid | (j << 8));
        }
    }
    return total;
}

}  // namespace tsv
