// gdn_large.hip -- gated-delta-rule verification over packed trees of 65 to
// 256 nodes ("TreeWY: Speculative Verification for Gated DeltaNet Hybrids",
// fugumt page, abstract: every draft node's output from one triangular solve
// over the tree). The same closed form as gdn.hip: with G_i the sum of g over
// the root path of i and D_ij = exp(G_i - G_j) (the sum of g over the path
// from i up to j, j excluded, accumulated along the walk),
//   e_i = beta_i (v_i - exp(G_i) S0 k_i) - beta_i sum_{j strict ancestor} D_ij (k_i . k_j) e_j,
//   o_i = exp(G_i) S0 q_i + sum_{j on path(i)} D_ij (q_i . k_j) e_j.
//
// Plain fp32 kernel, one 1024-thread work-group per (item, head):
//  1. tree check, depth, and every node's ancestor list (itself first, then
//     up to the root) in LDS; a tree with more than kGdnLargePairs
//     ancestor-or-self pairs is reported with status 8 and left untouched;
//  2. per pair, the partial log decay along the list, the key score
//     D_ij (k_i . k_j) and the query score D_ij (q_i . k_j) (dot products over
//     dk from the rows in memory);
//  3. per (node, 16 value rows) the right-hand side r_i, written to the
//     caller's e buffer, which holds the pseudo-values while they are solved
//     (S0 is staged in LDS transposed, and the lanes of a wave take the same
//     value rows of consecutive nodes, so every S0 read is a broadcast);
//  4. the solve one depth level at a time (a node's ancestors are on earlier
//     levels), in place in e;
//  5. per (node, 16 value rows) the output o_i.
// q, k, v and o are fp32 or bf16 (bits); g, beta, S0 and e fp32.
#include "common.hpp"
#include "launch.hpp"
#include "verify_common.hpp"

namespace tsv {

namespace {

constexpr int kGdnLargeNT = kMaxNodesLarge;  // threads (the tree work uses the first T)
constexpr int kGdnLargePairs = 4096;       // ancestor-or-self pairs held in LDS
constexpr int kGdnLargeDim = 128;          // dk, dv at most
constexpr int kGdnStOverCapacity = 8;
constexpr int kRowBlock = 16;              // value rows per work item

template <typename TIO, bool VEC>
__global__ __launch_bounds__(kGdnLargeNT) void gdn_large_kernel(
    const TIO* __restrict__ q, const TIO* __restrict__ k, const TIO* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ S0,
    const int32_t* __restrict__ parent, TIO* __restrict__ o, float* __restrict__ e,
    int32_t* __restrict__ tree_status, int T, int H, int dk, int dv) {
    constexpr int NT = kGdnLargeNT, MAXP = kGdnLargePairs;
    __shared__ int s_par[kMaxNodes];
    __shared__ int s_dep[kMaxNodes];
    __shared__ int s_off[kMaxNodes];
    __shared__ int s_scratch[kMaxNodes];
    __shared__ int s_scan[NT / kWave];
    __shared__ uint16_t s_pair[MAXP];  // node i in the low byte, ancestor j in the high byte
    __shared__ float s_ld[MAXP];       // log decay from j to i (j excluded)
    __shared__ float s_ak[MAXP];       // D_ij (k_i . k_j), 0 for j = i
    __shared__ float s_aq[MAXP];       // D_ij (q_i . k_j)
    __shared__ float s_gv[kMaxNodes];  // g of each node
    __shared__ float s_bt[kMaxNodes];  // beta of each node
    __shared__ float s_gam[kMaxNodes]; // exp(G_i)
    __shared__ int s_lvl[kMaxNodes];   // nodes ordered by depth
    __shared__ int s_lvs[kMaxNodes + 1];
    __shared__ int s_cnt[kMaxNodes];
    __shared__ int s_maxdep;
    __shared__ __align__(16) float s_S0t[kGdnLargeDim * kGdnLargeDim];  // S0 transposed: [c][p]

    const int b = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x;
    const size_t row0 = (size_t)b * T * H + h;  // (b, node 0, h) in units of a node's row
    const float* S0h = S0 + ((size_t)b * H + h) * dv * dk;

    // ---- 1. tree
    const int par_i = load_parent(parent + (size_t)b * T, T);
    float gi = 0.f, bi = 0.f;
    if (tid < T) {
        gi = g[row0 + (size_t)tid * H];
        bi = beta[row0 + (size_t)tid * H];
    }
    const int st = check_tree(par_i, T, s_par);
    if (st) {
        if (h == 0 && tid == 0 && tree_status) tree_status[b] = st;
        return;
    }
    const int total = build_pairs<NT>(s_par, T, s_dep, s_off, s_scratch, s_scan, s_pair, MAXP);
    if (total > MAXP) {
        if (h == 0 && tid == 0 && tree_status) tree_status[b] = kGdnStOverCapacity;
        return;
    }
    if (h == 0 && tid == 0 && tree_status) tree_status[b] = 0;
    if (tid < T) {
        s_gv[tid] = gi;
        s_bt[tid] = bi;
        s_cnt[tid] = 0;
    }
    if (tid == 0) s_maxdep = 0;
    for (int x = tid; x < dv * dk; x += NT) {
        const int pp = x / dk, c = x - pp * dk;
        s_S0t[c * dv + pp] = S0h[x];
    }
    __syncthreads();

    // ---- 2. partial log decays along each list, exp(G_i), depth counts
    if (tid < T) {
        const int base = s_off[tid], cnt = s_dep[tid] + 1;
        float part = 0.f;
        for (int m = 0; m < cnt; ++m) {
            s_ld[base + m] = part;
            part += s_gv[s_pair[base + m] >> 8];
        }
        s_gam[tid] = __expf(part);
        atomicAdd(&s_cnt[cnt - 1], 1);
        atomicMax(&s_maxdep, cnt - 1);
    }
    __syncthreads();
    const int maxdep = s_maxdep;
    if (tid == 0) {
        int run = 0;
        for (int d = 0; d <= maxdep; ++d) {
            s_lvs[d] = run;
            run += s_cnt[d];
            s_cnt[d] = s_lvs[d];  // next free slot of level d
        }
        s_lvs[maxdep + 1] = run;
    }
    __syncthreads();
    if (tid < T) s_lvl[atomicAdd(&s_cnt[s_dep[tid]], 1)] = tid;
    // pair scores, one pair per thread at a time
    for (int idx = tid; idx < total; idx += NT) {
        const int pr = s_pair[idx];
        const int i = pr & 255, j = pr >> 8;
        const TIO* ki = k + (row0 + (size_t)i * H) * dk;
        const TIO* kj = k + (row0 + (size_t)j * H) * dk;
        const TIO* qi = q + (row0 + (size_t)i * H) * dk;
        float kk = 0.f, qk = 0.f;
#pragma unroll 4
        for (int c = 0; c < dk; c += 4) {
            const float4 a = ld4io<TIO, VEC>(ki + c, dk - c), bj = ld4io<TIO, VEC>(kj + c, dk - c),
                         qq = ld4io<TIO, VEC>(qi + c, dk - c);
            kk += (a.x * bj.x + a.y * bj.y) + (a.z * bj.z + a.w * bj.w);
            qk += (qq.x * bj.x + qq.y * bj.y) + (qq.z * bj.z + qq.w * bj.w);
        }
        const float D = __expf(s_ld[idx]);
        s_ak[idx] = i == j ? 0.f : D * kk;
        s_aq[idx] = D * qk;
    }

    // ---- 3. right-hand sides r_i = beta_i (v_i - exp(G_i) S0 k_i) into e
    const int nrb = (dv + kRowBlock - 1) / kRowBlock;
    // S0 x (16 value rows from p0) for node i's row x_i: x_i from memory, S0 from LDS
    auto s0_rows = [&](const TIO* xi, int p0, float* acc) {
#pragma unroll
        for (int u = 0; u < kRowBlock; ++u) acc[u] = 0.f;
#pragma unroll 2
        for (int c0 = 0; c0 < dk; c0 += 4) {
            const float4 x4 = ld4io<TIO, VEC>(xi + c0, dk - c0);
            const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                if (c0 + cc >= dk) break;
                const float* sc = s_S0t + (c0 + cc) * dv + p0;
#pragma unroll
                for (int u = 0; u < kRowBlock; ++u)
                    if (p0 + u < dv) acc[u] += sc[u] * xs[cc];
            }
        }
    };
    // items (row block, node): the lanes of a wave share the row block
    for (int it = tid; it < T * nrb; it += NT) {
        const int pb = it / T, i = it - pb * T, p0 = pb * kRowBlock;
        float acc[kRowBlock];
        s0_rows(k + (row0 + (size_t)i * H) * dk, p0, acc);
        const size_t ro = (row0 + (size_t)i * H) * dv;
#pragma unroll
        for (int u = 0; u < kRowBlock; ++u) {
            const int p = p0 + u;
            if (p < dv) e[ro + p] = s_bt[i] * (Elem<TIO>::ld(v, ro + p) - s_gam[i] * acc[u]);
        }
    }
    __syncthreads();  // e holds r; the pair scores and levels are complete

    // ---- 4. the solve, level by level (the root's e is its r)
    for (int d = 1; d <= maxdep; ++d) {
        const int lo = s_lvs[d], items = (s_lvs[d + 1] - lo) * dv;
        for (int it = tid; it < items; it += NT) {
            const int n = it / dv, p = it - n * dv;
            const int i = s_lvl[lo + n];
            const int base = s_off[i], cnt = s_dep[i] + 1;
            const size_t ro = (row0 + (size_t)i * H) * dv;
            float acc = 0.f;
            for (int m0 = 1; m0 < cnt; m0 += 8) {  // eight ancestors' values in flight
                float ev[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int m = min(m0 + u, cnt - 1);
                    ev[u] = e[(row0 + (size_t)(s_pair[base + m] >> 8) * H) * dv + p];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (m0 + u < cnt) acc += s_ak[base + m0 + u] * ev[u];
            }
            e[ro + p] -= s_bt[i] * acc;
        }
        __syncthreads();
    }

    // ---- 5. outputs o_i = exp(G_i) S0 q_i + sum_{j on path(i)} D_ij (q_i . k_j) e_j
    for (int it = tid; it < T * nrb; it += NT) {
        const int pb = it / T, i = it - pb * T, p0 = pb * kRowBlock;
        float acc[kRowBlock];
        s0_rows(q + (row0 + (size_t)i * H) * dk, p0, acc);
        const int base = s_off[i], cnt = s_dep[i] + 1;
        const size_t ro = (row0 + (size_t)i * H) * dv;
#pragma unroll
        for (int u = 0; u < kRowBlock; ++u) {
            const int p = p0 + u;
            if (p >= dv) continue;
            float val = s_gam[i] * acc[u];
            for (int m0 = 0; m0 < cnt; m0 += 8) {
                float ev[8];
#pragma unroll
                for (int w8 = 0; w8 < 8; ++w8) {
                    const int m = min(m0 + w8, cnt - 1);
                    ev[w8] = e[(row0 + (size_t)(s_pair[base + m] >> 8) * H) * dv + p];
                }
#pragma unroll
                for (int w8 = 0; w8 < 8; ++w8)
                    if (m0 + w8 < cnt) val += s_aq[base + m0 + w8] * ev[w8];
            }
            Elem<TIO>::st(o, ro + p, val);
        }
    }
}

}  // namespace

bool gdn_large_supported(int T) { return T > 64 && T <= kMaxNodes; }

hipError_t launch_gdn_large(int batch, int T, int H, int dk, int dv, bool bf16, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, const float* S0,
                            const int32_t* parent, void* o, float* e, int32_t* tree_status, hipStream_t stream) {
    // vector loads of q and k rows: rows of a multiple of four elements, 16-byte
    // (fp32) or 8-byte (bf16) aligned
    const bool vec = dk % 4 == 0 && (((uintptr_t)q | (uintptr_t)k) & (bf16 ? 7 : 15)) == 0;
#define TSV_GDN_L(TIO, V)                                                                            \
    hipLaunchKernelGGL((gdn_large_kernel<TIO, V>), dim3(batch * H), dim3(kGdnLargeNT), 0, stream,   \
                       (const TIO*)q, (const TIO*)k, (const TIO*)v, g, beta, S0, parent, (TIO*)o, e, \
                       tree_status, T, H, dk, dv)
    if (bf16) {
        if (vec) TSV_GDN_L(uint16_t, true);
        else TSV_GDN_L(uint16_t, false);
    } else {
        if (vec) TSV_GDN_L(float, true);
        else TSV_GDN_L(float, false);
    }
#undef TSV_GDN_L
    return hipGetLastError();
}

}  // namespace tsv
