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
// fp32 throughout; trees of up to 64 nodes, dk and dv up to 128.
// Verify: one work-group of 512 threads (8 waves) per (item, head); wave w owns
// value rows [16 w, 16 w + 16) from the dense products to the outputs.
//  1. Every load is issued on entry: each wave's S0 rows straight into
//     registers (the B operand of its products), k and q for LDS, v in the
//     layout of the product accumulators. Meanwhile wave 0 alone (one lane per
//     node, no block barrier) checks the tree and finds by pointer jumping each
//     node's ancestor set (a 64-bit mask) and G_i, then lists the nodes by depth.
//  2. fp32 MFMA (16x16x4): K S0^T and Q S0^T per wave (nodes x its value rows);
//     the pair scores K K^T and Q K^T on the lower-triangle 16x16 tiles.
//  3. The pair-score tiles become two dense node x node matrices in LDS:
//     A_ij = beta_i D_ij (k_i . k_j) on strict ancestors and W_ij = D_ij (q_i . k_j)
//     on the path, D_ij = exp(G_i - G_j); each wave writes its right-hand sides
//     beta_i (v_i - exp(G_i) S0 k_i) into e.
//  4. The solve runs level by level inside each wave (the unknowns of a value
//     row depend only on the same row), four nodes of a level at a time.
//  5. o = exp(G) * (Q S0^T) + W e on MFMA, again per wave.
// Commit: one work-group per (item, head, 4,096-element chunk of the state),
// as for the SSD commit, reading the pseudo-values the verify call wrote.
#include "common.hpp"
#include "launch.hpp"
#include "verify_common.hpp"

namespace tsv {

constexpr int kGdnNodes = 64;
constexpr int kGdnDim = 128;
constexpr int kGdnThreads = 512;
constexpr int kGdnKS = kGdnDim + 4;    // row stride (floats) of staged k and q, and of e
constexpr int kGdnCS = kGdnNodes + 4;  // row stride of the coefficient matrices A and W
constexpr int kGdnStage = 2 * kGdnNodes * kGdnKS;                     // k, q
constexpr int kGdnPost = 2 * kGdnNodes * kGdnCS + kGdnNodes * kGdnKS;  // A, W, e
constexpr int kGdnUnion = kGdnStage > kGdnPost ? kGdnStage : kGdnPost;

// four consecutive floats of a row with `rem` >= 1 valid elements left (VEC: a
// 16-byte aligned row of a multiple of four elements)
template <bool VEC>
__device__ __forceinline__ float4 ld4(const float* __restrict__ p, int rem) {
    if (VEC) return *(const float4*)p;
    float4 r;
    r.x = p[0];
    r.y = rem > 1 ? p[1] : 0.f;
    r.z = rem > 2 ? p[2] : 0.f;
    r.w = rem > 3 ? p[3] : 0.f;
    return r;
}

__device__ __forceinline__ f32x4 mfma4(const float4& a, const float4& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
}

template <bool VEC>
__global__ __launch_bounds__(kGdnThreads) void gdn_verify_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ S0,
    const int32_t* __restrict__ parent, float* __restrict__ o, float* __restrict__ e_out,
    int32_t* __restrict__ tree_status, int T, int H, int dk, int dv) {
    constexpr int KS = kGdnKS, CS = kGdnCS;
    __shared__ __align__(16) float s_u[kGdnUnion];
    __shared__ unsigned long long s_mask[kGdnNodes];  // ancestors of i, i included
    __shared__ float s_G[kGdnNodes];
    __shared__ float s_gam[kGdnNodes];  // exp(G_i)
    __shared__ float s_beta[kGdnNodes];
    __shared__ int s_lvl[kGdnNodes];      // nodes by depth
    __shared__ int s_lvs[kGdnNodes + 1];  // start of each depth in s_lvl
    __shared__ int s_info[2];             // tree status, maximum depth
    float* const s_k = s_u;
    float* const s_q = s_u + kGdnNodes * KS;
    float* const s_A = s_u;  // after the products
    float* const s_W = s_u + kGdnNodes * CS;
    float* const s_e = s_u + 2 * kGdnNodes * CS;

    const int b = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane & 15, q4 = lane >> 4;
    const int NTI = (T + 15) >> 4;  // 16-node tiles
    const int nkk = (dk + 15) >> 4;  // 16-column steps over dk
    const size_t row0 = (size_t)b * T * H + h;  // (b, node 0, h) in units of a node's row
    const int p = 16 * w + l16;                  // value row of this lane
    const bool wave_rows = 16 * w < dv;          // wave-uniform

    // ---- 1. loads
    int par = 0;
    float gl = 0.f, bl = 0.f;
    if (w == 0) {
        const int i = min(lane, T - 1);
        par = parent[(size_t)b * T + i];
        gl = g[row0 + (size_t)i * H];
        bl = beta[row0 + (size_t)i * H];
    }
    float4 kst[4], qst[4];  // (node, 4 columns) slots of k and q, 32 slots per row
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int slot = tid + kGdnThreads * m, r = slot >> 5, c = 4 * (slot & 31);
        kst[m] = qst[m] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < T && c < dk) {
            const size_t src = (row0 + (size_t)r * H) * dk + c;
            kst[m] = ld4<VEC>(k + src, dk - c);
            qst[m] = ld4<VEC>(q + src, dk - c);
        }
    }
    // S0[p][16 kk + 4 q4 .. + 3]: lane (l16, q4) supplies columns 16 kk + 4 q4 + c
    // of the contraction over dk at step (kk, c)
    float4 s0r[kGdnDim / 16];
    const float* S0p = S0 + (((size_t)b * H + h) * dv + min(p, dv - 1)) * dk;
#pragma unroll
    for (int kk = 0; kk < kGdnDim / 16; ++kk) {
        const int col = 16 * kk + 4 * q4;
        s0r[kk] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (wave_rows && p < dv && col < dk) s0r[kk] = ld4<VEC>(S0p + col, dk - col);
    }
    // v at the accumulator positions: node 16 ti + 4 q4 + r, value row p
    float vr[kGdnNodes / 4];
#pragma unroll
    for (int ti = 0; ti < kGdnNodes / 16; ++ti)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * ti + 4 * q4 + r;
            vr[4 * ti + r] =
                wave_rows && i < T && p < dv ? v[(row0 + (size_t)i * H) * dv + p] : 0.f;
        }

    // ---- tree set-up by wave 0, one lane per node
    if (w == 0) {
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
            int start = 0;
            for (int d = 0; d <= maxdep; ++d) {
                const unsigned long long bm = __ballot(dep == d);
                if (dep == d) s_lvl[start + __popcll(bm & ((1ull << lane) - 1))] = lane;
                if (lane == 0) s_lvs[d] = start;
                start += __popcll(bm);
            }
            if (lane == 0) {
                s_lvs[maxdep + 1] = start;
                s_info[1] = maxdep;
            }
            s_mask[lane] = msk;
            s_G[lane] = G;
            s_gam[lane] = live ? __expf(G) : 0.f;
            s_beta[lane] = live ? bl : 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int slot = tid + kGdnThreads * m, r = slot >> 5, c = 4 * (slot & 31);
        *(float4*)&s_k[r * KS + c] = kst[m];
        *(float4*)&s_q[r * KS + c] = qst[m];
    }
    lds_barrier();
    if (s_info[0]) return;

    // ---- 2. products
    f32x4 R4[kGdnNodes / 16], Q4[kGdnNodes / 16];
#pragma unroll
    for (int ti = 0; ti < kGdnNodes / 16; ++ti) R4[ti] = Q4[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave_rows) {
#pragma unroll
        for (int ti = 0; ti < kGdnNodes / 16; ++ti) {
            if (ti < NTI) {
                const float* ka = s_k + (16 * ti + l16) * KS + 4 * q4;
                const float* qa = s_q + (16 * ti + l16) * KS + 4 * q4;
#pragma unroll
                for (int kk = 0; kk < kGdnDim / 16; ++kk) {
                    if (kk < nkk) {
                        R4[ti] = mfma4(*(const float4*)(ka + 16 * kk), s0r[kk], R4[ti]);
                        Q4[ti] = mfma4(*(const float4*)(qa + 16 * kk), s0r[kk], Q4[ti]);
                    }
                }
            }
        }
    }
    // pair scores on the lower-triangle tiles: tile t < ntri of K K^T, then of Q K^T
    const int ntri = NTI * (NTI + 1) / 2;
    constexpr int kPT = 3;  // tiles per wave: 2 * 10 lower-triangle tiles over 8 waves
    f32x4 P4[kPT];
    int pti[kPT], ptj[kPT];
#pragma unroll
    for (int u = 0; u < kPT; ++u) {
        P4[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int t = w + (kGdnThreads / kWave) * u;
        int ti = 0, tj = t < 2 * ntri ? t % ntri : -1;
        while (tj > ti) tj -= ++ti;
        pti[u] = ti;
        ptj[u] = tj;
        if (tj >= 0) {
            const float* xa = (t < ntri ? s_k : s_q) + (16 * ti + l16) * KS + 4 * q4;
            const float* kb = s_k + (16 * tj + l16) * KS + 4 * q4;
#pragma unroll
            for (int kk = 0; kk < kGdnDim / 16; ++kk)
                if (kk < nkk)
                    P4[u] = mfma4(*(const float4*)(xa + 16 * kk), *(const float4*)(kb + 16 * kk), P4[u]);
        }
    }
    lds_barrier();  // k and q consumed: the region now holds A, W and e

    // ---- 3. coefficients and right-hand sides
#pragma unroll
    for (int u = 0; u < kPT; ++u) {
        const int t = w + (kGdnThreads / kWave) * u;
        if (ptj[u] >= 0) {
            const int j = 16 * ptj[u] + l16;
            const float Gj = s_G[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * pti[u] + 4 * q4 + r;
                const bool anc = (s_mask[i] >> j) & 1ull;  // j on the root path of i
                const float D = __expf(s_G[i] - Gj);
                if (t < ntri)
                    s_A[i * CS + j] = anc && j != i ? s_beta[i] * D * P4[u][r] : 0.f;
                else
                    s_W[i * CS + j] = anc ? D * P4[u][r] : 0.f;
            }
        }
    }
    if (wave_rows) {
#pragma unroll
        for (int ti = 0; ti < kGdnNodes / 16; ++ti) {
            if (ti < NTI) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * ti + 4 * q4 + r;
                    s_e[i * KS + p] =
                        i < T ? s_beta[i] * (vr[4 * ti + r] - s_gam[i] * R4[ti][r]) : 0.f;
                }
            }
        }
    }
    lds_barrier();
    if (!wave_rows) return;

    // ---- 4. solve, level by level within the wave
    const int maxdep = s_info[1];
    for (int d = 0; d <= maxdep; ++d) {
        const int hi = s_lvs[d + 1];
        for (int pos = s_lvs[d] + q4; pos < hi; pos += 4) {
            const int i = s_lvl[pos];
            unsigned long long m = s_mask[i] & ~(1ull << i);
            float acc = s_e[i * KS + p];
            while (m) {
                int j[4];
                bool ok[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ok[u] = m != 0ull;
                    j[u] = ok[u] ? (int)__builtin_ctzll(m) : 0;
                    m &= m - 1ull;
                }
                float a[4], x[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    a[u] = s_A[i * CS + j[u]];
                    x[u] = s_e[j[u] * KS + p];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = ok[u] ? acc - a[u] * x[u] : acc;
            }
            s_e[i * KS + p] = acc;
            if (e_out && p < dv) e_out[(row0 + (size_t)i * H) * dv + p] = acc;
        }
        wave_sync();
    }

    // ---- 5. outputs: o = exp(G) (Q S0^T) + W e, tiles below the diagonal only
#pragma unroll
    for (int ti = 0; ti < kGdnNodes / 16; ++ti) {
        if (ti < NTI) {
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = s_gam[16 * ti + 4 * q4 + r] * Q4[ti][r];
            for (int tj = 0; tj <= ti; ++tj) {
                const float4 wv = *(const float4*)&s_W[(16 * ti + l16) * CS + 16 * tj + 4 * q4];
                const float* ep = s_e + (16 * tj + 4 * q4) * KS + p;
                const float4 ev = make_float4(ep[0], ep[KS], ep[2 * KS], ep[3 * KS]);
                acc = mfma4(wv, ev, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + 4 * q4 + r;
                if (i < T && p < dv) o[(row0 + (size_t)i * H) * dv + p] = acc[r];
            }
        }
    }
}

constexpr int kGdnPathChunk = 16;

__global__ __launch_bounds__(kBlock) void gdn_commit_kernel(
    const float* __restrict__ k, const float* __restrict__ g, const float* __restrict__ e,
    float* __restrict__ S, const int32_t* __restrict__ parent, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ accepted_len, int32_t* __restrict__ tree_status, int T, int H,
    int dk, int dv, int Lmax, int chunks) {
    __shared__ int s_par[kMaxNodes];
    __shared__ int s_path[kMaxNodes];
    __shared__ float s_w[kMaxNodes];
    __shared__ float s_w0;
    __shared__ float s_e[kGdnPathChunk][kGdnDim];
    __shared__ float s_k[kGdnPathChunk][kGdnDim];
    const int chunk = blockIdx.x % chunks;
    const int bh = blockIdx.x / chunks;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    const int PN = dv * dk;
    const size_t row0 = (size_t)b * T * H + h;
    const int len = accepted_len[b];
    const int acc_i = Lmax > 0 ? accepted[(size_t)b * Lmax + min(tid, Lmax - 1)] : 0;
    const int par_i = load_parent(parent + (size_t)b * T, T);
    float* Sh = S + ((size_t)b * H + h) * PN;
    constexpr int kEl = 16;  // state elements per thread
    float acc[kEl];
    const int e0 = chunk * kBlock * kEl;
#pragma unroll
    for (int m = 0; m < kEl; ++m) {
        const int x = e0 + m * kBlock + tid;
        acc[m] = x < PN ? Sh[x] : 0.f;
    }
    const bool len_ok = len >= 0 && len <= Lmax;
    if (len_ok && tid < len) s_path[tid] = acc_i;
    int st = check_tree(par_i, T, s_par);
    int bad = 0;
    if (!st) {
        if (!len_ok) {
            bad = 1;
        } else if (tid < len) {
            const int node = s_path[tid];
            bad = tid == 0 ? node != 0 : (node < 0 || node >= T || s_par[node] != s_path[tid - 1]);
        }
    }
    if (__syncthreads_or(bad)) st |= kStBadPath;
    if (h == 0 && chunk == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st || len == 0) return;
    // decay weights along the path: w_t = exp(sum of g after entry t), w0 = exp(sum of all)
    if (tid < len) s_w[tid] = g[row0 + (size_t)s_path[tid] * H];
    __syncthreads();
    if (tid == 0) {
        float c = 0.f;
        for (int t = len - 1; t >= 0; --t) {
            const float gt = s_w[t];
            s_w[t] = __expf(c);
            c += gt;
        }
        s_w0 = __expf(c);
    }
    __syncthreads();
    const float w0 = s_w0;
#pragma unroll
    for (int m = 0; m < kEl; ++m) acc[m] *= w0;
    for (int t0 = 0; t0 < len; t0 += kGdnPathChunk) {
        const int tn = min(kGdnPathChunk, len - t0);
        if (t0 > 0) __syncthreads();
        for (int x = tid; x < tn * dv; x += kBlock) {
            const int t = x / dv, p = x % dv;
            s_e[t][p] = s_w[t0 + t] * e[(row0 + (size_t)s_path[t0 + t] * H) * dv + p];
        }
        for (int x = tid; x < tn * dk; x += kBlock) {
            const int t = x / dk, n = x % dk;
            s_k[t][n] = k[(row0 + (size_t)s_path[t0 + t] * H) * dk + n];
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < kEl; ++m) {
            const int x = e0 + m * kBlock + tid;
            if (x < PN) {
                const int p = x / dk, n = x % dk;
                float a = acc[m];
                for (int t = 0; t < tn; ++t) a += s_e[t][p] * s_k[t][n];
                acc[m] = a;
            }
        }
    }
#pragma unroll
    for (int m = 0; m < kEl; ++m) {
        const int x = e0 + m * kBlock + tid;
        if (x < PN) Sh[x] = acc[m];
    }
}

hipError_t launch_gdn_verify(int batch, int T, int H, int dk, int dv, const float* q,
                             const float* k, const float* v, const float* g, const float* beta,
                             const float* S0, const int32_t* parent, float* o, float* e,
                             int32_t* tree_status, hipStream_t stream) {
    const bool vec = dk % 4 == 0 && (((uintptr_t)q | (uintptr_t)k | (uintptr_t)S0) & 15) == 0;
    if (vec)
        hipLaunchKernelGGL(gdn_verify_kernel<true>, dim3(batch * H), dim3(kGdnThreads), 0, stream,
                           q, k, v, g, beta, S0, parent, o, e, tree_status, T, H, dk, dv);
    else
        hipLaunchKernelGGL(gdn_verify_kernel<false>, dim3(batch * H), dim3(kGdnThreads), 0, stream,
                           q, k, v, g, beta, S0, parent, o, e, tree_status, T, H, dk, dv);
    return hipGetLastError();
}

hipError_t launch_gdn_commit(int batch, int T, int H, int dk, int dv, const float* k,
                             const float* g, const float* e, float* S, const int32_t* parent,
                             const int32_t* accepted, const int32_t* accepted_len, int Lmax,
                             int32_t* tree_status, hipStream_t stream) {
    const int per_wg = kBlock * 16;
    const int chunks = (dv * dk + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(gdn_commit_kernel, dim3(batch * H * chunks), dim3(kBlock), 0, stream, k, g,
                       e, S, parent, accepted, accepted_len, tree_status, T, H, dk, dv, Lmax,
                       chunks);
    return hipGetLastError();
}

}  // namespace tsv
