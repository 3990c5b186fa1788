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
// Verify: one work-group of 512 threads per (item, head). Set-up: tree check,
// depth and ancestor-pair lists in LDS, decays along each list. Then dk is
// walked in chunks of 32 columns staged in LDS (S0 columns, k and q rows): the
// pair scores k_i . k_j and q_i . k_j accumulate per pair, the dense products
// K S0^T and Q S0^T (nodes x value rows) on fp32 MFMA (16x16x4), each wave
// owning whole 16 x 16 output tiles; a lane's (node, value-row) units are the
// MFMA output elements it holds, so they stay in registers for the solve. The solve runs
// depth level by depth level (a barrier per level): every unit of the level
// sums over its node's strict ancestors' pseudo-values in LDS. The outputs sum
// over the whole path.
// Commit: one work-group per (item, head, 4,096-element chunk of the state),
// as for the SSD commit, reading the pseudo-values the verify call wrote.
#include "common.hpp"
#include "launch.hpp"
#include "verify_common.hpp"

namespace tsv {

constexpr int kGdnNodes = 64;
constexpr int kGdnDim = 128;
constexpr int kGdnThreads = 512;
constexpr int kGdnChunk = 32;                          // dk columns staged at a time
constexpr int kGdnPairs = kGdnNodes * (kGdnNodes + 1) / 2;
constexpr int kGdnTilesPW = (kGdnNodes / 16) * (kGdnDim / 16) / (kGdnThreads / kWave);  // 16x16 output tiles per wave
constexpr int kGdnUnits = 4 * kGdnTilesPW;  // (node, value-row) units per lane
constexpr int kGdnPairsPT = (kGdnPairs + kGdnThreads - 1) / kGdnThreads;

__global__ __launch_bounds__(kGdnThreads) void gdn_verify_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ S0,
    const int32_t* __restrict__ parent, float* __restrict__ o, float* __restrict__ e_out,
    int32_t* __restrict__ tree_status, int T, int H, int dk, int dv) {
    constexpr int KC = kGdnChunk;
    __shared__ int s_par[kMaxNodes];
    __shared__ int s_dep[kMaxNodes];
    __shared__ int s_off[kMaxNodes];
    __shared__ int s_scratch[kMaxNodes];
    __shared__ int s_scan[kGdnThreads / kWave];
    __shared__ uint16_t s_pair[kGdnPairs];
    __shared__ float s_KK[kGdnPairs];  // k_i . k_j
    __shared__ float s_QK[kGdnPairs];  // q_i . k_j
    __shared__ float s_D[kGdnPairs];   // exp(G_i - G_j)
    __shared__ float s_gam[kGdnNodes];  // exp(G_i)
    __shared__ float s_g[kGdnNodes];
    __shared__ float s_beta[kGdnNodes];
    __shared__ float s_S0c[kGdnDim][KC + 1];
    __shared__ float s_kc[kGdnNodes][KC + 1];
    __shared__ float s_qc[kGdnNodes][KC + 1];
    __shared__ float s_e[kGdnNodes][kGdnDim];
    __shared__ int s_maxdep;

    const int b = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x;
    const size_t row0 = (size_t)b * T * H + h;  // (b, node 0, h) in units of a node's row
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane & 15, q4 = lane >> 4;
    const int NTI = (T + 15) / 16, NTP = (dv + 15) / 16;  // node tiles, value-row tiles
    // unit m of this lane: output tile tt = w + 8 (m / 4), element row 4 q4 + m % 4,
    // column l16; node i = 16 (tt / NTP) + 4 q4 + m % 4, value row p = 16 (tt % NTP) + l16
    auto unit = [&](int m, int& i, int& p) {
        const int tt = w + (kGdnThreads / kWave) * (m >> 2);
        i = 16 * (tt / NTP) + 4 * q4 + (m & 3);
        p = 16 * (tt % NTP) + l16;
        return tt < NTI * NTP && i < T && p < dv;
    };
    const int par_i = load_parent(parent + (size_t)b * T, T);
    float vr[kGdnUnits];
#pragma unroll
    for (int m = 0; m < kGdnUnits; ++m) {
        int i, p;
        unit(m, i, p);
        vr[m] = v[(row0 + (size_t)min(i, T - 1) * H) * dv + min(p, dv - 1)];
    }
    const int st = check_tree(par_i, T, s_par);
    if (h == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st) return;
    if (tid < T) {
        s_g[tid] = g[row0 + (size_t)tid * H];
        s_beta[tid] = beta[row0 + (size_t)tid * H];
    }
    if (tid == 0) s_maxdep = 0;
    const int total = build_pairs<kGdnThreads>(s_par, T, s_dep, s_off, s_scratch, s_scan, s_pair,
                                               kGdnPairs);
    (void)total;  // every tree of up to 64 nodes fits
    // decays along each node's list (entry 0 is the node itself)
    if (tid < T) {
        const int base = s_off[tid], cnt = s_dep[tid] + 1;
        float s = 0.f;
        for (int kk = 0; kk < cnt; ++kk) {
            const int j = s_pair[base + kk] >> 8;
            s_D[base + kk] = __expf(s);
            s += s_g[j];
        }
        s_gam[tid] = __expf(s);
        atomicMax(&s_maxdep, cnt - 1);
    }
    // dk in chunks: pair scores per pair, S0 k_i and S0 q_i per (node, row) unit
    float kk_acc[kGdnPairsPT], qk_acc[kGdnPairsPT];
    f32x4 R4[kGdnTilesPW], Q4[kGdnTilesPW];
#pragma unroll
    for (int m = 0; m < kGdnPairsPT; ++m) kk_acc[m] = qk_acc[m] = 0.f;
#pragma unroll
    for (int t = 0; t < kGdnTilesPW; ++t) R4[t] = Q4[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* S0h = S0 + ((size_t)b * H + h) * dv * dk;
    for (int c0 = 0; c0 < dk; c0 += KC) {
        const int wc = min(KC, dk - c0);
        __syncthreads();  // previous chunk consumed (and, the first time, the set-up done)
        for (int x = tid; x < 16 * NTP * KC; x += kGdnThreads) {
            const int p = x / KC, n = x % KC;
            s_S0c[p][n] = n < wc && p < dv ? S0h[(size_t)p * dk + c0 + n] : 0.f;
        }
        for (int x = tid; x < 16 * NTI * KC; x += kGdnThreads) {
            const int i = x / KC, n = x % KC;
            const size_t src = (row0 + (size_t)i * H) * dk + c0 + n;
            s_kc[i][n] = n < wc && i < T ? k[src] : 0.f;
            s_qc[i][n] = n < wc && i < T ? q[src] : 0.f;
        }
        __syncthreads();
        const int npairs = s_off[T - 1] + s_dep[T - 1] + 1;
#pragma unroll
        for (int m = 0; m < kGdnPairsPT; ++m) {
            const int pq = tid + kGdnThreads * m;
            if (pq < npairs) {
                const int pr = s_pair[pq];
                const int i = pr & 255, j = pr >> 8;
                float a = 0.f, c = 0.f;
#pragma unroll 8
                for (int n = 0; n < KC; ++n) {
                    a += s_kc[i][n] * s_kc[j][n];
                    c += s_qc[i][n] * s_kc[j][n];
                }
                kk_acc[m] += a;
                qk_acc[m] += c;
            }
        }
        // D[node][row] += sum_n K[node][n] S0[row][n]: A = K (lane l16 = node,
        // q4 = k), B = S0^T (q4 = k, l16 = row); same for Q
#pragma unroll
        for (int t = 0; t < kGdnTilesPW; ++t) {
            const int tt = w + (kGdnThreads / kWave) * t;
            if (tt < NTI * NTP) {
                const int ni = 16 * (tt / NTP) + l16, pr = 16 * (tt % NTP) + l16;
#pragma unroll
                for (int ks = 0; ks < KC / 4; ++ks) {
                    const float bs = s_S0c[pr][4 * ks + q4];
                    R4[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(s_kc[ni][4 * ks + q4], bs, R4[t], 0, 0, 0);
                    Q4[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(s_qc[ni][4 * ks + q4], bs, Q4[t], 0, 0, 0);
                }
            }
        }
    }
    float R[kGdnUnits], Q0[kGdnUnits];
#pragma unroll
    for (int m = 0; m < kGdnUnits; ++m) {
        R[m] = R4[m >> 2][m & 3];
        Q0[m] = Q4[m >> 2][m & 3];
    }
    {
        const int npairs = s_off[T - 1] + s_dep[T - 1] + 1;
#pragma unroll
        for (int m = 0; m < kGdnPairsPT; ++m) {
            const int pq = tid + kGdnThreads * m;
            if (pq < npairs) {
                s_KK[pq] = kk_acc[m];
                s_QK[pq] = qk_acc[m];
            }
        }
    }
    __syncthreads();
    // triangular solve, one depth level at a time
    const int maxdep = s_maxdep;
    for (int d = 0; d <= maxdep; ++d) {
#pragma unroll
        for (int m = 0; m < kGdnUnits; ++m) {
            int i, p;
            if (unit(m, i, p)) {
                if (s_dep[i] == d) {
                    const int base = s_off[i];
                    float acc = 0.f;
                    for (int kk = 1; kk <= d; ++kk) {
                        const int j = s_pair[base + kk] >> 8;
                        acc += s_D[base + kk] * s_KK[base + kk] * s_e[j][p];
                    }
                    const float bi = s_beta[i];
                    s_e[i][p] = bi * (vr[m] - s_gam[i] * R[m]) - bi * acc;
                }
            }
        }
        __syncthreads();
    }
    // outputs over the whole path, and the pseudo-values for commit
#pragma unroll
    for (int m = 0; m < kGdnUnits; ++m) {
        int i, p;
        if (unit(m, i, p)) {
            const int base = s_off[i], cnt = s_dep[i] + 1;
            float acc = s_gam[i] * Q0[m];
            for (int kk = 0; kk < cnt; ++kk) {
                const int j = s_pair[base + kk] >> 8;
                acc += s_D[base + kk] * s_QK[base + kk] * s_e[j][p];
            }
            const size_t dst = (row0 + (size_t)i * H) * dv + p;
            o[dst] = acc;
            if (e_out) e_out[dst] = s_e[i][p];
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
    hipLaunchKernelGGL(gdn_verify_kernel, dim3(batch * H), dim3(kGdnThreads), 0, stream, q, k, v,
                       g, beta, S0, parent, o, e, tree_status, T, H, dk, dv);
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
