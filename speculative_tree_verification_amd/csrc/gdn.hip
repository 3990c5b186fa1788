// gdn.hip -- packed-tree verification and commit for the gated delta rule
// ("TreeWY: Speculative Verification for Gated DeltaNet Hybrids", fugumt page,
// abstract: every draft node's output from one triangular solve over the tree,
// and only the accepted state rebuilt on commit from a pseudo-value matrix).
// Per head, state S (dv x dk, stored [p][n]), token inputs q, k (dk), v (dv),
// log gate g and step beta:
//   S <- exp(g) S (I - beta k k^T) + beta v k^T,   o = S q,
// run from S0 along each node's root path. With G_i the sum of g over the root
// path of i and D_ij = exp(G_i - G_j) (summed along the path from i up to j,
// not formed as a difference), the pseudo-values e solve
//   e_i + beta_i sum_{j strict ancestor} D_ij (k_i . k_j) e_j = beta_i (v_i - exp(G_i) S0 k_i)
// (a unit lower-triangular system restricted to ancestors, so each node's row
// involves its own root path only), and
//   o_i = exp(G_i) S0 q_i + sum_{j on path(i)} D_ij (q_i . k_j) e_j,
//   S'  = exp(G_l) S0 + sum_{j on path(l)} D_lj e_j k_j^T   (commit, path to l).
//
// q, k, v and o fp32 or bf16 (bits); g, beta, S0 and the pseudo-values e
// fp32; trees of up to 64 nodes, dk and dv up to 128. bf16 rows of q and k go
// to LDS as their bits: they are the exact high part, with no low part to
// stage or multiply (their products with S0 take two terms, their pair scores
// one).
// Verify: one work-group of 9 waves per (item, head). Row wave w < 8 owns value
// rows [16 w, 16 w + 16); the tree wave handles everything node x node.
//  1. Every load is issued on entry: each row wave's S0 rows straight into
//     registers (the B operand of its products), k and q for LDS (split into
//     bf16 high and low parts), v in the layout of the product accumulators.
//     Meanwhile the tree wave (one lane per node) checks the tree and finds by
//     pointer jumping each node's ancestor set (a 64-bit mask) and G_i, and
//     lists each node's strict ancestors by depth.
//  2. Row waves: K S0^T and Q S0^T (nodes x its value rows) on MFMA with
//     three-term bf16 splits (hi*hi + hi*lo + lo*hi, fp32 accumulation), then the
//     right-hand sides r_i = beta_i (v_i - exp(G_i) S0 k_i) in registers.
//     Tree wave, at the same time: the pair scores K K^T and Q K^T on the
//     lower-triangle 16x16 tiles (same splits), A_ij = beta_i D_ij (k_i . k_j) on
//     strict ancestors, W_ij = D_ij (q_i . k_j) on the path (D_ij = exp(G_i - G_j)),
//     and M = (I + A)^{-1} row by row from M (I + A) = I, one lane a row, each
//     entry from the row's entries nearer to its node (no sync per depth
//     level): M is ancestor-masked like A, and it is shared by every value row.
//  3. Row waves: e = M r and o = exp(G) * (Q S0^T) + W e on fp32 MFMA; the
//     accumulators of r and e are laid out as the B operand of the next product,
//     so they never leave registers.
// Commit: one work-group per (item, head, 4,096-element chunk of the state),
// as for the SSD commit, reading the pseudo-values the verify call wrote.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "verify_common.hpp"

namespace tsv {

constexpr int kGdnNodes = 64;
constexpr int kGdnDim = 128;
constexpr int kGdnRowWaves = 8;  // row wave w owns value rows [16 w, 16 w + 16)
constexpr int kGdnRowThreads = kGdnRowWaves * kWave;
constexpr int kGdnThreads = kGdnRowThreads + kWave;  // and the tree wave
constexpr int kGdnRS = kGdnDim + 8;    // row stride (bf16) of the staged halves of k and q
constexpr int kGdnCS = kGdnNodes + 4;  // row stride of the dense node x node matrices

// x = hi + lo for four floats: bf16 high parts and bf16 residuals, packed in pairs
__device__ __forceinline__ void split4(const float4& x, uint2& hi, uint2& lo) {
    const uint32_t h01 = pack_bf16x2(x.x, x.y), h23 = pack_bf16x2(x.z, x.w);
    hi = make_uint2(h01, h23);
    lo = make_uint2(pack_bf16x2(x.x - lo_bf16(h01), x.y - hi_bf16(h01)),
                    pack_bf16x2(x.z - lo_bf16(h23), x.w - hi_bf16(h23)));
}

// a b with both operands split into bf16 high and low parts: the three products
// hi*hi + hi*lo + lo*hi accumulate in fp32 (about 16 significant bits per operand)
__device__ __forceinline__ f32x4 mfma_x3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                         const bf16x8& bl, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
}

// a b with a exact in bf16 (a bf16 input row) and b split: hi*lo + hi*hi
__device__ __forceinline__ f32x4 mfma_x2(const bf16x8& ah, const bf16x8& bh, const bf16x8& bl, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
}

// four consecutive bf16 elements of a row as bits (zero past the row's end)
template <bool VEC>
__device__ __forceinline__ uint2 ld4bits(const uint16_t* __restrict__ p, int rem) {
    if (VEC) return gload((const uint2*)p);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int t = 0; t < 4; ++t)
        if (t < rem) w[t >> 1] |= (uint32_t)gload(p + t) << (16 * (t & 1));
    return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ f32x4 mfma4(const float4& a, const float4& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
}

template <typename TIO, bool VEC>
__global__ __launch_bounds__(kGdnThreads) void gdn_verify_kernel(
    const TIO* __restrict__ q, const TIO* __restrict__ k, const TIO* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ S0,
    const int32_t* __restrict__ parent, TIO* __restrict__ o, float* __restrict__ e_out,
    int32_t* __restrict__ tree_status, int T, int H, int dk, int dv) {
    constexpr int NN = kGdnNodes, RS = kGdnRS, CS = kGdnCS;
    constexpr bool SVEC = VEC;  // the launch checks S0's alignment with the rows'
    __shared__ __align__(16) uint16_t s_stage[4 * NN * RS];  // k hi, k lo, q hi, q lo
    __shared__ __align__(16) float s_A[NN * NN];  // A_ij at [i][depth of j]
    __shared__ __align__(16) float s_W[NN * CS];
    __shared__ __align__(16) float s_M[NN * CS];
    __shared__ __align__(16) uint8_t s_anc[NN * NN];  // strict ancestors of i, root first
    __shared__ unsigned long long s_mask[NN];          // ancestors of i, i included
    __shared__ float s_G[NN];
    __shared__ float s_gam[NN];  // exp(G_i)
    __shared__ float s_beta[NN];
    __shared__ int s_dep[NN];
    __shared__ int s_info[1];      // tree status
    uint16_t* const s_kh = s_stage;
    uint16_t* const s_kl = s_kh + NN * RS;
    uint16_t* const s_qh = s_kl + NN * RS;
    uint16_t* const s_ql = s_qh + NN * RS;

    const int b = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane & 15, q4 = lane >> 4;
    const int NTI = (T + 15) >> 4;   // 16-node tiles
    const int nks = (dk + 31) >> 5;  // 32-column steps over dk
    const size_t row0 = (size_t)b * T * H + h;  // (b, node 0, h) in units of a node's row
    const bool tree_wave = w == kGdnRowWaves;
    const int p = 16 * w + l16;                    // value row of this lane (row waves)
    const bool wave_rows = !tree_wave && 16 * w < dv;  // wave-uniform

    // ---- 1. loads
    int par = 0;
    float gl = 0.f, bl = 0.f;
    if (tree_wave) {
        const int i = min(lane, T - 1);
        par = parent[(size_t)b * T + i];
        gl = g[row0 + (size_t)i * H];
        bl = beta[row0 + (size_t)i * H];
    }
    // (node, 4 columns) slots of k and q, 32 slots per row: fp32 rows as
    // floats (split into bf16 parts for LDS), bf16 rows as their bits (exact
    // in the high part; no low part is staged or multiplied)
    constexpr bool BF = sizeof(TIO) == 2;
    float4 kst[4], qst[4];
    uint2 kbits[4], qbits[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int slot = tid + kGdnRowThreads * m, r = slot >> 5, c = 4 * (slot & 31);
        kst[m] = qst[m] = make_float4(0.f, 0.f, 0.f, 0.f);
        kbits[m] = qbits[m] = make_uint2(0u, 0u);
        if (!tree_wave && r < T && c < dk) {
            const size_t src = (row0 + (size_t)r * H) * dk + c;
            if constexpr (BF) {
                kbits[m] = ld4bits<VEC>((const uint16_t*)k + src, dk - c);
                qbits[m] = ld4bits<VEC>((const uint16_t*)q + src, dk - c);
            } else {
                kst[m] = ld4io<TIO, VEC>(k + src, dk - c);
                qst[m] = ld4io<TIO, VEC>(q + src, dk - c);
            }
        }
    }
    if (tree_wave) {
        // ---- tree set-up, one lane per node
        const bool live = lane < T;
        const bool br = __ballot(lane == 0 && par != -1) != 0;
        const bool bp = __ballot(live && lane > 0 && (par < 0 || par >= lane)) != 0;
        const int st = (br ? kStBadRoot : 0) | (bp ? kStBadParent : 0);
        if (lane == 0) {
            s_info[0] = st;
            if (h == 0 && tree_status) tree_status[b] = st;
        }
        if (!st) {
            // pointer jumping: lane i covers the path from i up to (not including)
            // n, its mask and its sum of g; merging with n's segment doubles it
            unsigned long long msk = live ? 1ull << lane : 0ull;
            int n = live && lane > 0 ? par : -1;
            float G = live ? gl : 0.f;
            while (__ballot(n >= 0)) {
                const int src = n >= 0 ? n : lane;
                const uint32_t mlo = __shfl((uint32_t)msk, src, kWave);
                const uint32_t mhi = __shfl((uint32_t)(msk >> 32), src, kWave);
                const int n2 = __shfl(n, src, kWave);
                const float G2 = __shfl(G, src, kWave);
                if (n >= 0) {
                    msk |= ((unsigned long long)mhi << 32) | mlo;
                    G += G2;
                    n = n2;
                }
            }
            const int dep = live ? __popcll(msk) - 1 : -1;
            int maxdep = dep;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) maxdep = max(maxdep, __shfl_xor(maxdep, off, kWave));
            // the strict ancestors of each node by depth: climb one step a round
            const int up = live && lane > 0 ? par : 0;
            int cur = lane;
            for (int t = 0; t < maxdep; ++t) {
                cur = __shfl(up, cur, kWave);
                if (t < dep) s_anc[lane * NN + dep - 1 - t] = (uint8_t)cur;
            }
            s_dep[lane] = live ? dep : 0;
            s_mask[lane] = msk;
            s_G[lane] = G;
            s_gam[lane] = live ? __expf(G) : 0.f;
            s_beta[lane] = live ? bl : 0.f;
        }
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int slot = tid + kGdnRowThreads * m, r = slot >> 5, c = 4 * (slot & 31);
            if constexpr (BF) {
                *(uint2*)&s_kh[r * RS + c] = kbits[m];
                *(uint2*)&s_qh[r * RS + c] = qbits[m];
            } else {
                uint2 hi, lo;
                split4(kst[m], hi, lo);
                *(uint2*)&s_kh[r * RS + c] = hi;
                *(uint2*)&s_kl[r * RS + c] = lo;
                split4(qst[m], hi, lo);
                *(uint2*)&s_qh[r * RS + c] = hi;
                *(uint2*)&s_ql[r * RS + c] = lo;
            }
        }
    }
    // S0 and v are requested only now, so that k and q (needed first) do not
    // share the memory system with them
    // S0[p][32 ks + 8 q4 .. + 7]: lane (l16, q4) supplies columns 32 ks + 8 q4 + c
    // of the contraction over dk at step ks
    float4 s0r[kGdnDim / 16];
    const float* S0p = S0 + (((size_t)b * H + h) * dv + min(p, dv - 1)) * dk;
#pragma unroll
    for (int kk = 0; kk < kGdnDim / 16; ++kk) {
        const int col = 32 * (kk >> 1) + 8 * q4 + 4 * (kk & 1);
        s0r[kk] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (wave_rows && p < dv && col < dk) s0r[kk] = ld4<SVEC>(S0p + col, dk - col);
    }
    // v at the accumulator positions: node 16 ti + 4 q4 + r, value row p
    float vr[NN / 4];
#pragma unroll
    for (int ti = 0; ti < NN / 16; ++ti)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * ti + 4 * q4 + r;
            vr[4 * ti + r] =
                wave_rows && i < T && p < dv ? Elem<TIO>::ld(v, (row0 + (size_t)i * H) * dv + p) : 0.f;
        }

    lds_barrier();
    if (s_info[0]) return;

    // ---- 2. pair scores on the lower-triangle tiles (tile t < ntri of K K^T,
    // then of Q K^T; three-term bf16 splits), coefficients A and W, M = I there
    const int ntri = NTI * (NTI + 1) / 2;
    if (!tree_wave) {
#pragma unroll
        for (int u = 0; u < 3; ++u) {  // 2 * 10 tiles at most over 8 waves
            const int t = w + kGdnRowWaves * u;
            if (t < 2 * ntri) {
                const bool kk = t < ntri;
                int ti = 0, tj = kk ? t : t - ntri;
                while (tj > ti) tj -= ++ti;
                const int oa = (16 * ti + l16) * RS + 8 * q4, ob = (16 * tj + l16) * RS + 8 * q4;
                const uint16_t* xh = kk ? s_kh : s_qh;
                const uint16_t* xl = kk ? s_kl : s_ql;
                f32x4 P = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < kGdnDim / 32; ++ks)
                    if (ks < nks)
                        P = BF ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(xh + oa + 32 * ks),
                                                                         *(const bf16x8*)(s_kh + ob + 32 * ks), P, 0,
                                                                         0, 0)
                               : mfma_x3(*(const bf16x8*)(xh + oa + 32 * ks), *(const bf16x8*)(xl + oa + 32 * ks),
                                         *(const bf16x8*)(s_kh + ob + 32 * ks), *(const bf16x8*)(s_kl + ob + 32 * ks),
                                         P);
                const int j = 16 * tj + l16;
                const float Gj = s_G[j];
                const int dj = s_dep[j];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * ti + 4 * q4 + r;
                    const bool anc = (s_mask[i] >> j) & 1ull;  // j on the root path of i
                    const float D = __expf(s_G[i] - Gj);
                    if (kk) {
                        if (anc && j != i) s_A[i * NN + dj] = s_beta[i] * D * P[r];
                        s_M[i * CS + j] = i == j ? 1.f : 0.f;
                    } else {
                        s_W[i * CS + j] = anc ? D * P[r] : 0.f;
                    }
                }
            }
        }
    }
    lds_barrier();

    f32x4 Q4[NN / 16], R4[NN / 16];  // Q S0^T, then the right-hand sides r
#pragma unroll
    for (int ti = 0; ti < NN / 16; ++ti) R4[ti] = Q4[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (tree_wave) {
        // ---- 3b. M, by the tree wave while the row waves form their products.
        // M (I + A) = I row by row: lane i takes row i, from its parent's depth
        // up to the root; for c the strict ancestor of i at depth t,
        //   M_ic = -A_ic - sum over the path nodes x strictly between c and i of M_ix A_xc,
        // each entry from the row's entries nearer to i (no sync per depth level)
        if (lane < T) {
            const int i = lane, d = s_dep[i];
            const uint8_t* an = s_anc + i * NN;
            const float* ai = s_A + i * NN;
            for (int t = d - 1; t >= 0; --t) {
                float acc = -ai[t];
                for (int s0 = t + 1; s0 < d; s0 += 4) {
                    float mv[4], av[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int x = an[min(s0 + u, d - 1)];
                        mv[u] = s_M[i * CS + x];
                        av[u] = s_A[x * NN + t];
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc = s0 + u < d ? acc - mv[u] * av[u] : acc;
                }
                s_M[i * CS + an[t]] = acc;
            }
        }
    } else if (wave_rows) {
        // ---- 3a. products (three-term bf16 splits, fp32 accumulation)
        bf16x8 s0h[kGdnDim / 32], s0l[kGdnDim / 32];
#pragma unroll
        for (int ks = 0; ks < kGdnDim / 32; ++ks) split_hi_lo(s0r[2 * ks], s0r[2 * ks + 1], s0h[ks], s0l[ks]);
#pragma unroll
        for (int ti = 0; ti < NN / 16; ++ti) {
            if (ti < NTI) {
                const int oa = (16 * ti + l16) * RS + 8 * q4;
#pragma unroll
                for (int ks = 0; ks < kGdnDim / 32; ++ks) {
                    if (ks < nks) {
                        const int c = oa + 32 * ks;
                        if constexpr (BF) {
                            R4[ti] = mfma_x2(*(const bf16x8*)(s_kh + c), s0h[ks], s0l[ks], R4[ti]);
                            Q4[ti] = mfma_x2(*(const bf16x8*)(s_qh + c), s0h[ks], s0l[ks], Q4[ti]);
                        } else {
                            R4[ti] = mfma_x3(*(const bf16x8*)(s_kh + c), *(const bf16x8*)(s_kl + c),
                                             s0h[ks], s0l[ks], R4[ti]);
                            Q4[ti] = mfma_x3(*(const bf16x8*)(s_qh + c), *(const bf16x8*)(s_ql + c),
                                             s0h[ks], s0l[ks], Q4[ti]);
                        }
                    }
                }
                // right-hand sides r_i = beta_i (v_i - exp(G_i) S0 k_i), 0 past the tree
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * ti + 4 * q4 + r;
                    R4[ti][r] = i < T ? s_beta[i] * (vr[4 * ti + r] - s_gam[i] * R4[ti][r]) : 0.f;
                }
            }
        }
    }
    lds_barrier();  // M and W complete
    if (!wave_rows) return;

    // ---- 4. e = M r, o = exp(G) (Q S0^T) + W e over the tiles below the diagonal.
    // The accumulator of a 16x16 tile holds (node 16 t + 4 q4 + c, row p) in
    // element c, which is the B operand of node 16 t + 4 q4 + c at k step c.
    f32x4 E4[NN / 16];
#pragma unroll
    for (int ti = 0; ti < NN / 16; ++ti) {
        E4[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (ti < NTI) {
#pragma unroll
            for (int tj = 0; tj <= ti; ++tj) {
                const float4 mv = *(const float4*)&s_M[(16 * ti + l16) * CS + 16 * tj + 4 * q4];
                E4[ti] = mfma4(mv, make_float4(R4[tj][0], R4[tj][1], R4[tj][2], R4[tj][3]), E4[ti]);
            }
        }
    }
    TIO* const o_p = o + row0 * dv + p;
    float* const e_p = e_out ? e_out + row0 * dv + p : nullptr;
    const size_t step = (size_t)H * dv;  // next node
#pragma unroll
    for (int ti = 0; ti < NN / 16; ++ti) {
        if (ti < NTI) {
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = s_gam[16 * ti + 4 * q4 + r] * Q4[ti][r];
#pragma unroll
            for (int tj = 0; tj <= ti; ++tj) {
                const float4 wv = *(const float4*)&s_W[(16 * ti + l16) * CS + 16 * tj + 4 * q4];
                acc = mfma4(wv, make_float4(E4[tj][0], E4[tj][1], E4[tj][2], E4[tj][3]), acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + 4 * q4 + r;
                if (i < T && p < dv) {
                    Elem<TIO>::st(o_p, (size_t)i * step, acc[r]);
                    if (e_p) e_p[(size_t)i * step] = E4[ti][r];
                }
            }
        }
    }
}

constexpr int kGdnCommitEl = kBlock * 16;                       // state elements per chunk
// State chunks per work-group. One is the fastest measured: 2 and 4 (the later
// chunks streamed behind the path rows, their stores overlapping the loads
// still in flight) leave fewer waves per CU and took 9% and 16% longer at
// batch 16, 16 heads, dk = dv = 128.
constexpr int kGdnCommitCPW = 1;

// Commit: S' = w0 S0 + sum_t w_t e_{j_t} k_{j_t}^T over the accepted path
// j_0 = 0, ..., j_{L-1}, with w_t = exp(sum of g after entry t) and w0 = exp(sum
// of all g on the path). One work-group per (item, head, CPW chunks of the
// state). The path indices, the parents and the first state chunk leave first; the tree and the path are
// validated with barriers that wait for LDS only, so that the next round trip
// (g of the path, the e and k rows) leaves at once, followed by the other state
// chunks; each chunk is then updated and written back as it arrives, its
// stores overlapping the loads still in flight. The weights come from a suffix
// scan across one wave.
template <typename TIO, bool VEC, int CPW>
__global__ __launch_bounds__(kBlock) void gdn_commit_kernel(
    const TIO* __restrict__ k, const float* __restrict__ g, const float* __restrict__ e,
    float* __restrict__ S, const int32_t* __restrict__ parent, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ accepted_len, int32_t* __restrict__ tree_status, int T, int H,
    int dk, int dv, int Lmax, int EW, int KW, int groups) {
    __shared__ int s_par[kMaxNodes];     // trees of up to 256 nodes
    __shared__ int s_path[kGdnMaxPath];  // paths of up to 128 nodes
    __shared__ int s_bad[kBlock / kWave];
    __shared__ float s_w[kGdnMaxPath];
    __shared__ float s_g[kGdnMaxPath];   // g of the path (paths past 64 nodes)
    __shared__ float s_w0;
    // [min(Lmax, T)][EW] e rows of the path, then [min(Lmax, T)][KW] k rows
    extern __shared__ __attribute__((aligned(16))) float s_dyn[];
    float* const s_e = s_dyn;
    float* const s_k = s_dyn + min(Lmax, T) * EW;
    const int grp = blockIdx.x % groups;
    const int b = blockIdx.x / groups / H, h = blockIdx.x / groups % H;
    const int tid = threadIdx.x;
    const int PN = dv * dk;
    const size_t row0 = (size_t)b * T * H + h;
    const int len = accepted_len[b];
    const int acc_i = Lmax > 0 ? accepted[(size_t)b * Lmax + min(tid, Lmax - 1)] : 0;
    const int par_i = load_parent(parent + (size_t)b * T, T);
    float* Sh = S + ((size_t)b * H + h) * PN;
    const int c0 = grp * CPW;  // first chunk of this work-group
    float4 acc[CPW][4];  // [chunk][piece]: elements (c0 + c) * 4096 + (v * 256 + tid) * 4 ..
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int pe = (c0 + c) * kGdnCommitEl + (v * kBlock + tid) * 4;
            if (VEC) {
                acc[c][v] = pe < PN ? *(const float4*)(Sh + pe) : make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
                acc[c][v].x = pe < PN ? Sh[pe] : 0.f;
                acc[c][v].y = pe + 1 < PN ? Sh[pe + 1] : 0.f;
                acc[c][v].z = pe + 2 < PN ? Sh[pe + 2] : 0.f;
                acc[c][v].w = pe + 3 < PN ? Sh[pe + 3] : 0.f;
            }
        }
    };
    load_chunk(0);

    // tree and path checks (a valid path starts at the root and steps from
    // parent to child, so its indices increase and len <= T)
    const bool len_ok = len >= 0 && len <= Lmax && len <= T;
    if (tid < T) s_par[tid] = par_i;
    if (len_ok && tid < len) s_path[tid] = acc_i;
    lds_barrier();
    int bits = 0;
    if (tid == 0 && par_i != -1) bits |= kStBadRoot;
    if (tid > 0 && tid < T && (par_i < 0 || par_i >= tid)) bits |= kStBadParent;
    if (!len_ok) {
        if (tid == 0) bits |= kStBadPath;
    } else if (tid < len) {
        const int node = s_path[tid];
        if (tid == 0 ? node != 0 : (node < 0 || node >= T || s_par[node] != s_path[tid - 1]))
            bits |= kStBadPath;
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) bits |= __shfl_xor(bits, off, kWave);
    if ((tid & (kWave - 1)) == 0) s_bad[tid / kWave] = bits;
    lds_barrier();
    int st = 0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) st |= s_bad[w];
    if (st & (kStBadRoot | kStBadParent)) st &= ~kStBadPath;  // a path is checked on a valid tree only
    if (h == 0 && grp == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st || len == 0) return;

    // one round trip: g of the path, the e and k rows; then the other chunks
    const float gt = tid < len ? g[row0 + (size_t)s_path[tid] * H] : 0.f;
    const int kq = VEC ? dk / 4 : dk;  // k pieces per row
    const int ne = len * dv, nk = len * kq;
    for (int base = 0; base < max(ne, nk); base += 4 * kBlock) {
        float ev[4];
        float4 kv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int x = base + u * kBlock + tid;
            ev[u] = 0.f;
            kv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (x < ne) {
                const int t = x / dv, r = x - t * dv;
                ev[u] = e[(row0 + (size_t)s_path[t] * H) * dv + r];
            }
            if (x < nk) {
                const int t = x / kq, c = x - t * kq;
                const TIO* src = k + (row0 + (size_t)s_path[t] * H) * dk;
                if (VEC)
                    kv[u] = ld4io<TIO, true>(src + 4 * c, 4);
                else
                    kv[u].x = Elem<TIO>::ld(src, c);
            }
        }
        if (base == 0) {
#pragma unroll
            for (int c = 1; c < CPW; ++c) load_chunk(c);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int x = base + u * kBlock + tid;
            if (x < ne) {
                const int t = x / dv;
                s_e[t * EW + x - t * dv] = ev[u];
            }
            if (x < nk) {
                const int t = x / kq, c = x - t * kq;
                if (VEC)
                    *(float4*)&s_k[t * KW + 4 * c] = kv[u];
                else
                    s_k[t * KW + c] = kv[u].x;
            }
        }
    }
    if (len <= kWave) {
        if (tid < kWave) {
            // w_t = exp(sum of g over entries after t): inclusive suffix scan of
            // the sequence shifted by one entry (len <= 64 lanes)
            float x = __shfl_down(gt, 1, kWave);
            if (tid == kWave - 1) x = 0.f;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float y = __shfl_down(x, off, kWave);
                if (tid + off < kWave) x += y;
            }
            if (tid < len) s_w[tid] = __expf(x);
            if (tid == 0) s_w0 = __expf(x + gt);
        }
    } else {
        // longer paths: each entry adds up the g after it
        if (tid < len) s_g[tid] = gt;
        lds_barrier();
        if (tid < len) {
            float x = 0.f;
            for (int t = tid + 1; t < len; ++t) x += s_g[t];
            s_w[tid] = __expf(x);
            if (tid == 0) s_w0 = __expf(x + gt);
        }
    }
    lds_barrier();
    const float w0 = s_w0;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        if ((c0 + c) * kGdnCommitEl >= PN) break;
        float4* a = acc[c];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            a[v].x *= w0;
            a[v].y *= w0;
            a[v].z *= w0;
            a[v].w *= w0;
        }
        const int pe0 = (c0 + c) * kGdnCommitEl + tid * 4;
        if (VEC && (kBlock * 4) % dk == 0) {
            // the four pieces of this thread cover the same columns n .. n+3 of
            // four rows: one k read per path entry serves all of them
            const int n = pe0 % dk;
            int pr[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) pr[v] = min((pe0 + v * kBlock * 4) / dk, dv - 1);
            for (int t = 0; t < len; ++t) {
                const float4 kk = *(const float4*)&s_k[t * KW + n];
                const float wt = s_w[t];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float ew = wt * s_e[t * EW + pr[v]];
                    a[v].x += ew * kk.x;
                    a[v].y += ew * kk.y;
                    a[v].z += ew * kk.z;
                    a[v].w += ew * kk.w;
                }
            }
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float f[4] = {a[v].x, a[v].y, a[v].z, a[v].w};
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int x = pe0 + v * kBlock * 4 + cc;
                    if (x < PN) {
                        const int pr = x / dk, n = x - pr * dk;
                        for (int t = 0; t < len; ++t) f[cc] += s_w[t] * s_e[t * EW + pr] * s_k[t * KW + n];
                    }
                }
                a[v] = make_float4(f[0], f[1], f[2], f[3]);
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int pe = pe0 + v * kBlock * 4;
            if (VEC) {
                if (pe < PN) *(float4*)(Sh + pe) = a[v];
            } else {
                if (pe < PN) Sh[pe] = a[v].x;
                if (pe + 1 < PN) Sh[pe + 1] = a[v].y;
                if (pe + 2 < PN) Sh[pe + 2] = a[v].z;
                if (pe + 3 < PN) Sh[pe + 3] = a[v].w;
            }
        }
    }
}

hipError_t launch_gdn_verify(int batch, int T, int H, int dk, int dv, bool bf16, const void* q,
                             const void* k, const void* v, const float* g, const float* beta,
                             const float* S0, const int32_t* parent, void* o, float* e,
                             int32_t* tree_status, hipStream_t stream) {
    // vector loads: rows of a multiple of four elements, q and k 16-byte (fp32)
    // or 8-byte (bf16) aligned, S0 16-byte aligned
    const uintptr_t ra = bf16 ? 7 : 15;
    const bool vec = dk % 4 == 0 && (((uintptr_t)q | (uintptr_t)k) & ra) == 0 && ((uintptr_t)S0 & 15) == 0;
#define TSV_GDN_V(TIO, V)                                                                              \
    hipLaunchKernelGGL((gdn_verify_kernel<TIO, V>), dim3(batch * H), dim3(kGdnThreads), 0, stream,     \
                       (const TIO*)q, (const TIO*)k, (const TIO*)v, g, beta, S0, parent, (TIO*)o, e, \
                       tree_status, T, H, dk, dv)
    if (bf16) {
        if (vec) TSV_GDN_V(uint16_t, true);
        else TSV_GDN_V(uint16_t, false);
    } else {
        if (vec) TSV_GDN_V(float, true);
        else TSV_GDN_V(float, false);
    }
#undef TSV_GDN_V
    return hipGetLastError();
}

hipError_t launch_gdn_commit(int batch, int T, int H, int dk, int dv, bool bf16, const void* k,
                             const float* g, const float* e, float* S, const int32_t* parent,
                             const int32_t* accepted, const int32_t* accepted_len, int Lmax,
                             int32_t* tree_status, hipStream_t stream) {
    // row strides of the staged e and k rows, in multiples of 4 floats
    const int EW = (dv + 3) / 4 * 4;
    const int KW = (dk + 3) / 4 * 4;
    const size_t shmem = (size_t)std::min(Lmax, T) * (EW + KW) * sizeof(float);
    const uintptr_t ra = bf16 ? 7 : 15;
    const bool vec = dk % 4 == 0 && ((uintptr_t)S & 15) == 0 && ((uintptr_t)k & ra) == 0;
    constexpr int CPW = kGdnCommitCPW;
    const int groups = ((dv * dk + kGdnCommitEl - 1) / kGdnCommitEl + CPW - 1) / CPW;
    const void* kern = bf16 ? (vec ? (const void*)gdn_commit_kernel<uint16_t, true, CPW>
                                   : (const void*)gdn_commit_kernel<uint16_t, false, CPW>)
                            : (vec ? (const void*)gdn_commit_kernel<float, true, CPW>
                                   : (const void*)gdn_commit_kernel<float, false, CPW>);
    if (shmem > 48 * 1024) {
        // paths of up to 128 entries with 128-wide rows take up to 128 KiB
        const hipError_t err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (err != hipSuccess) return err;
    }
    void* args[] = {(void*)&k, (void*)&g, (void*)&e, (void*)&S, (void*)&parent, (void*)&accepted,
                    (void*)&accepted_len, (void*)&tree_status, (void*)&T, (void*)&H, (void*)&dk,
                    (void*)&dv, (void*)&Lmax, (void*)&EW, (void*)&KW, (void*)&groups};
    return hipLaunchKernel(kern, dim3(batch * H * groups), dim3(kBlock), args, shmem, stream);
}

}  // namespace tsv
