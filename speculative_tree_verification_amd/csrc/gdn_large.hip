// gdn_large.hip -- gated-delta-rule verification over packed trees of 65 to
// 256 nodes ("TreeWY: Speculative Verification for Gated DeltaNet Hybrids",
// fugumt page, abstract: every draft node's output from one triangular solve
// over the tree). The same closed form as gdn.hip: with G_i the sum of g over
// the root path of i and D_ij = exp(G_i - G_j) (the sum of g over the path
// from i up to j, j excluded, accumulated along the walk),
//   r_i = beta_i (v_i - exp(G_i) S0 k_i),
//   e_i + sum_{j strict ancestor} A_ij e_j = r_i,   A_ij = beta_i D_ij (k_i . k_j),
//   o_i = exp(G_i) S0 q_i + sum_{j on path(i)} W_ij e_j,   W_ij = D_ij (q_i . k_j).
// With M = (I + A)^{-1} and N = W M, both nonzero on ancestor-or-self pairs
// only, e = M r and o = exp(G) S0 q + N r: the solve moves from the value rows
// onto one scalar per pair, and both outputs come from one gather over r.
//
// One work-group of 16 waves per (item, head); wave w owns nodes [16 w, 16 w + 16):
//  1. tree check, depth and every node's ancestor list (itself first, then up
//     to the root) in LDS; a tree with more than kGdnLargePairs
//     ancestor-or-self pairs is reported with status 8 and left untouched.
//     S0 is staged in LDS as bf16 high and low parts, in the order the MFMA B
//     operand reads it (one linear 1 KB read per wave and step).
//  2. K S0^T for the wave's 16 nodes on MFMA (three-term bf16 splits, fp32
//     accumulation; two terms for bf16 inputs, whose low parts are zero), then
//     r into the caller's e buffer; Q S0^T stays in registers. The column
//     order of the product tiles gives each lane four consecutive value rows
//     twice, so v, r, e and o move as 16-byte vectors.
//  3. pair scores, eight lanes per pair (k_i, k_j and q_i rows from memory);
//     M by substitution one depth level at a time, one pair entry per thread:
//        M_ij = -A_ij - sum_{x strictly between j and i} A_ix M_xj;
//     then N_ij = sum_{x from i down to j} W_ix M_xj, all entries at once.
//  4. e_i = sum_j M_ij r_j and o_i = exp(G_i) (S0 q_i) + sum_j N_ij r_j over the
//     root path of i, reading r back from e; e is written once every wave has
//     read r.
// q, k, v and o are fp32 or bf16 (bits); g, beta, S0 and e fp32.
#include "common.hpp"
#include "launch.hpp"
#include "verify_common.hpp"

namespace tsv {

namespace {

constexpr int kGdnLargeNT = 1024;      // 16 waves, 16 nodes each
constexpr int kGdnLargePairs = 4096;   // ancestor-or-self pairs held in LDS
constexpr int kGdnLargeDim = 128;      // dk, dv at most
constexpr int kGdnStOverCapacity = 8;
constexpr int kLNB = kGdnLargeDim / 16;  // column blocks of the S0 products
constexpr int kLKS = kGdnLargeDim / 32;  // contraction steps of 32 over dk
constexpr int kS0Ent = kLNB * kLKS * kWave;  // B-operand entries (8 values each)

// Value row held in column c of product column block nb: lane l16 (= c) owns
// rows 4 l16 .. 4 l16 + 3 (blocks 0..3) and 64 + 4 l16 .. + 3 (blocks 4..7).
__device__ __forceinline__ int vrow(int nb, int c) { return 64 * (nb >> 2) + 4 * c + (nb & 3); }

__device__ __forceinline__ f32x4 mfma_hl3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                          const bf16x8& bl, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_hl2(const bf16x8& ah, const bf16x8& bh, const bf16x8& bl, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
}

// four consecutive floats to a row of TIO elements (rem of them left in the row)
template <typename TIO, bool VEC>
__device__ __forceinline__ void st4io(TIO* __restrict__ p, const float4& x, int rem) {
    if constexpr (sizeof(TIO) == 4) {
        if (VEC) {
            gstore((float4*)p, x);
        } else {
            p[0] = x.x;
            if (rem > 1) p[1] = x.y;
            if (rem > 2) p[2] = x.z;
            if (rem > 3) p[3] = x.w;
        }
    } else {
        if (VEC) {
            gstore((uint2*)p, make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w)));
        } else {
            Elem<TIO>::st(p, 0, x.x);
            if (rem > 1) Elem<TIO>::st(p, 1, x.y);
            if (rem > 2) Elem<TIO>::st(p, 2, x.z);
            if (rem > 3) Elem<TIO>::st(p, 3, x.w);
        }
    }
}

// The 16 x 32 A operand of step ks for the wave's nodes: lane (l16, q4) holds
// columns 32 ks + 8 q4 .. + 7 of node row `row` (zero past dk or past the tree)
template <typename TIO, bool VEC>
__device__ __forceinline__ void load_a(const TIO* __restrict__ row, bool live, int q4, int dk, float4* a) {
#pragma unroll
    for (int ks = 0; ks < kLKS; ++ks) {
        const int c = 32 * ks + 8 * q4;
        a[2 * ks] = a[2 * ks + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live && c < dk) a[2 * ks] = ld4io<TIO, VEC>(row + c, dk - c);
        if (live && c + 4 < dk) a[2 * ks + 1] = ld4io<TIO, VEC>(row + c + 4, dk - c - 4);
    }
}

// X S0^T for the wave's 16 nodes: acc[nb] holds (node 16 w + 4 q4 + r, value
// row vrow(nb, l16)) in element r
template <bool BF>
__device__ __forceinline__ void s0_product(const float4* a, const bf16x8* __restrict__ s_S0, int lane, int dk,
                                           int dv, f32x4* acc) {
#pragma unroll
    for (int nb = 0; nb < kLNB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kLKS; ++ks) {
        if (32 * ks >= dk) break;
        bf16x8 ah, al;
        split_hi_lo(a[2 * ks], a[2 * ks + 1], ah, al);
#pragma unroll
        for (int nb = 0; nb < kLNB; ++nb) {
            if (vrow(nb, 0) >= dv) continue;
            const int x = (nb * kLKS + ks) * kWave + lane;
            const bf16x8 bh = s_S0[x], bl = s_S0[kS0Ent + x];
            acc[nb] = BF ? mfma_hl2(ah, bh, bl, acc[nb]) : mfma_hl3(ah, al, bh, bl, acc[nb]);
        }
    }
}

template <typename TIO, bool VEC>
__global__ __launch_bounds__(kGdnLargeNT) void gdn_large_kernel(
    const TIO* __restrict__ q, const TIO* __restrict__ k, const TIO* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ S0,
    const int32_t* __restrict__ parent, TIO* __restrict__ o, float* __restrict__ e,
    int32_t* __restrict__ tree_status, int T, int H, int dk, int dv) {
    constexpr int NT = kGdnLargeNT, MAXP = kGdnLargePairs;
    constexpr bool BF = sizeof(TIO) == 2;
    __shared__ int s_par[kMaxNodes];
    __shared__ int s_dep[kMaxNodes];
    __shared__ int s_off[kMaxNodes];
    __shared__ int s_scratch[kMaxNodes];
    __shared__ int s_red[NT / kWave];
    __shared__ uint16_t s_pair[MAXP];  // node i in the low byte, ancestor j in the high byte
    __shared__ uint16_t s_aof[MAXP];   // start of the list of j
    __shared__ float s_A[MAXP];        // log decay, then A_ij (0 at j = i), then N_ij
    __shared__ float s_W[MAXP];        // W_ij
    __shared__ float s_M[MAXP];        // M_ij (1 at j = i)
    __shared__ float s_gv[kMaxNodes];  // g of each node
    __shared__ float s_bt[kMaxNodes];  // beta of each node
    __shared__ float s_gam[kMaxNodes]; // exp(G_i)
    __shared__ int s_lvl[kMaxNodes];   // nodes ordered by depth
    __shared__ int s_lvs[kMaxNodes + 1];
    __shared__ int s_cnt[kMaxNodes];
    __shared__ int s_maxdep;
    __shared__ bf16x8 s_S0[2 * kS0Ent];  // S0 high parts, then low parts, in B-operand order

    const int b = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane & 15, q4 = lane >> 4;
    const size_t row0 = (size_t)b * T * H + h;  // (b, node 0, h) in units of a node's row
    const float* S0h = S0 + ((size_t)b * H + h) * dv * dk;
    const bool rows = 16 * w < T;  // wave-uniform: the wave owns nodes

    // ---- 1. loads, tree
    const int par_i = load_parent(parent + (size_t)b * T, T);
    float gi = 0.f, bi = 0.f;
    if (tid < T) {
        gi = g[row0 + (size_t)tid * H];
        bi = beta[row0 + (size_t)tid * H];
    }
    float4 s0v[4];  // B-operand entries tid and tid + NT: S0[vrow(nb, l16')][32 ks + 8 q4' .. + 7]
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int x = tid + NT * u, ln = x & (kWave - 1), ks = (x / kWave) % kLKS, nb = x / (kWave * kLKS);
        const int p = vrow(nb, ln & 15), c = 32 * ks + 8 * (ln >> 4);
        s0v[2 * u] = s0v[2 * u + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p < dv && c < dk) s0v[2 * u] = ld4<VEC>(S0h + (size_t)p * dk + c, dk - c);
        if (p < dv && c + 4 < dk) s0v[2 * u + 1] = ld4<VEC>(S0h + (size_t)p * dk + c + 4, dk - c - 4);
    }
    const int ia = 16 * w + l16;  // A-operand row of this lane
    const bool alive = rows && ia < T;
    float4 ka[2 * kLKS];
    load_a<TIO, VEC>(k + (row0 + (size_t)min(ia, T - 1) * H) * dk, alive, q4, dk, ka);

    const int st = check_tree_lds<NT>(par_i, T, s_par, s_red);
    if (st) {
        if (h == 0 && tid == 0 && tree_status) tree_status[b] = st;
        return;
    }
    const int total = build_pairs<NT>(s_par, T, s_dep, s_off, s_scratch, s_red, s_pair, MAXP);
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
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        bf16x8 hi, lo;
        split_hi_lo(s0v[2 * u], s0v[2 * u + 1], hi, lo);
        s_S0[tid + NT * u] = hi;
        s_S0[kS0Ent + tid + NT * u] = lo;
    }
    lds_barrier();

    // partial log decays along each list, exp(G_i), list starts, M_ii, depth counts
    if (tid < T) {
        const int base = s_off[tid], cnt = s_dep[tid] + 1;
        float part = 0.f;
        for (int m = 0; m < cnt; ++m) {
            const int j = s_pair[base + m] >> 8;
            s_A[base + m] = part;
            s_aof[base + m] = (uint16_t)s_off[j];
            part += s_gv[j];
        }
        s_M[base] = 1.f;
        s_gam[tid] = __expf(part);
        atomicAdd(&s_cnt[cnt - 1], 1);
        atomicMax(&s_maxdep, cnt - 1);
    }
    lds_barrier();
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
    lds_barrier();
    if (tid < T) s_lvl[atomicAdd(&s_cnt[s_dep[tid]], 1)] = tid;

    // ---- 2. K S0^T -> r into e; Q S0^T kept
    f32x4 qs[kLNB];
    if (rows) {
        const int i4 = 16 * w + 4 * q4;  // nodes i4 .. i4 + 3 of this lane's accumulators
        float4 vv[8];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int i = i4 + r, p0 = 64 * hf + 4 * l16;
                vv[2 * r + hf] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (i < T && p0 < dv) vv[2 * r + hf] = ld4io<TIO, VEC>(v + (row0 + (size_t)i * H) * dv + p0, dv - p0);
            }
        f32x4 ks_[kLNB];
        s0_product<BF>(ka, s_S0, lane, dk, dv, ks_);
        float4 qa[2 * kLKS];
        load_a<TIO, VEC>(q + (row0 + (size_t)min(ia, T - 1) * H) * dk, alive, q4, dk, qa);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i4 + r;
            if (i >= T) continue;
            const float bt = s_bt[i], gm = s_gam[i];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int p0 = 64 * hf + 4 * l16;
                if (p0 >= dv) continue;
                const float4 x = vv[2 * r + hf];
                const float4 rr = make_float4(bt * (x.x - gm * ks_[4 * hf][r]), bt * (x.y - gm * ks_[4 * hf + 1][r]),
                                              bt * (x.z - gm * ks_[4 * hf + 2][r]),
                                              bt * (x.w - gm * ks_[4 * hf + 3][r]));
                st4io<float, VEC>(e + (row0 + (size_t)i * H) * dv + p0, rr, dv - p0);
            }
        }
        s0_product<BF>(qa, s_S0, lane, dk, dv, qs);
    }

    // ---- 3. pair scores, eight lanes per pair (lane part: columns 16 sub .. + 15)
    {
        const int sub = lane & 7;
        const int rounds = (total + NT / 8 - 1) / (NT / 8);
        for (int rd = 0; rd < rounds; ++rd) {
            const int idx = rd * (NT / 8) + (tid >> 3);
            float kk = 0.f, qk = 0.f;
            int i = 0;
            if (idx < total) {
                const int pr = s_pair[idx];
                i = pr & 255;
                const int j = pr >> 8, c0 = 16 * sub;
                const TIO* ki = k + (row0 + (size_t)i * H) * dk + c0;
                const TIO* kj = k + (row0 + (size_t)j * H) * dk + c0;
                const TIO* qi = q + (row0 + (size_t)i * H) * dk + c0;
                float4 a[4], bj[4], qq[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    a[u] = bj[u] = qq[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (c0 + 4 * u < dk) {
                        a[u] = ld4io<TIO, VEC>(ki + 4 * u, dk - c0 - 4 * u);
                        bj[u] = ld4io<TIO, VEC>(kj + 4 * u, dk - c0 - 4 * u);
                        qq[u] = ld4io<TIO, VEC>(qi + 4 * u, dk - c0 - 4 * u);
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    kk += (a[u].x * bj[u].x + a[u].y * bj[u].y) + (a[u].z * bj[u].z + a[u].w * bj[u].w);
                    qk += (qq[u].x * bj[u].x + qq[u].y * bj[u].y) + (qq[u].z * bj[u].z + qq[u].w * bj[u].w);
                }
            }
#pragma unroll
            for (int off = 1; off < 8; off <<= 1) {
                kk += __shfl_xor(kk, off, kWave);
                qk += __shfl_xor(qk, off, kWave);
            }
            if (idx < total && sub == 0) {
                const float D = __expf(s_A[idx]);
                s_A[idx] = idx > s_off[i] ? s_bt[i] * D * kk : 0.f;
                s_W[idx] = D * qk;
            }
        }
    }
    lds_barrier();

    // M, one depth level at a time: entry (i, m) for the ancestor m steps up
    for (int d = 1; d <= maxdep; ++d) {
        const int lo = s_lvs[d], entries = (s_lvs[d + 1] - lo) * d;
        for (int x = tid; x < entries; x += NT) {
            const int ni = x / d, m = 1 + x - ni * d;
            const int base = s_off[s_lvl[lo + ni]];
            float acc = -s_A[base + m];
            for (int m0 = 1; m0 < m; m0 += 4) {
                float a[4], mv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int mm = min(m0 + u, m - 1);  // x = the ancestor mm steps up
                    a[u] = s_A[base + mm];
                    mv[u] = s_M[s_aof[base + mm] + m - mm];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (m0 + u < m) acc -= a[u] * mv[u];
            }
            s_M[base + m] = acc;
        }
        lds_barrier();
    }
    // N = W M over every pair (A is no longer needed)
    for (int x = tid; x < total; x += NT) {
        const int base = s_off[s_pair[x] & 255], m = x - base;
        float acc = 0.f;
        for (int m0 = 0; m0 <= m; m0 += 4) {
            float wv[4], mv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int mm = min(m0 + u, m);
                wv[u] = s_W[base + mm];
                mv[u] = s_M[s_aof[base + mm] + m - mm];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (m0 + u <= m) acc += wv[u] * mv[u];
        }
        s_A[x] = acc;
    }
    __syncthreads();  // N complete, and every wave's r is in e

    // ---- 4. e = M r, o = exp(G) (Q S0^T) + N r over each root path
    float4 ea[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * q4 + r;
        ea[2 * r] = ea[2 * r + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (!rows || i >= T) continue;
        const float gm = s_gam[i];
        float4 oa[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            oa[hf] = make_float4(gm * qs[4 * hf][r], gm * qs[4 * hf + 1][r], gm * qs[4 * hf + 2][r],
                                 gm * qs[4 * hf + 3][r]);
        const int base = s_off[i], cnt = s_dep[i] + 1;
        for (int m0 = 0; m0 < cnt; m0 += 4) {
            float4 rv[4][2];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = s_pair[base + min(m0 + u, cnt - 1)] >> 8;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int p0 = 64 * hf + 4 * l16;
                    rv[u][hf] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (p0 < dv) rv[u][hf] = ld4<VEC>(e + (row0 + (size_t)j * H) * dv + p0, dv - p0);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (m0 + u >= cnt) break;
                const float mv = s_M[base + m0 + u], nv = s_A[base + m0 + u];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float4 x = rv[u][hf];
                    ea[2 * r + hf].x += mv * x.x;
                    ea[2 * r + hf].y += mv * x.y;
                    ea[2 * r + hf].z += mv * x.z;
                    ea[2 * r + hf].w += mv * x.w;
                    oa[hf].x += nv * x.x;
                    oa[hf].y += nv * x.y;
                    oa[hf].z += nv * x.z;
                    oa[hf].w += nv * x.w;
                }
            }
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int p0 = 64 * hf + 4 * l16;
            if (p0 < dv) st4io<TIO, VEC>(o + (row0 + (size_t)i * H) * dv + p0, oa[hf], dv - p0);
        }
    }
    __syncthreads();  // every wave has read r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * q4 + r;
        if (!rows || i >= T) continue;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int p0 = 64 * hf + 4 * l16;
            if (p0 < dv) st4io<float, VEC>(e + (row0 + (size_t)i * H) * dv + p0, ea[2 * r + hf], dv - p0);
        }
    }
}

}  // namespace

bool gdn_large_supported(int T) { return T > 64 && T <= kMaxNodes; }

hipError_t launch_gdn_large(int batch, int T, int H, int dk, int dv, bool bf16, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, const float* S0,
                            const int32_t* parent, void* o, float* e, int32_t* tree_status, hipStream_t stream) {
    // 16-byte moves of fp32 rows (8-byte of bf16 rows): rows of a multiple of
    // four elements, every row array aligned to the move
    const uintptr_t io = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o;
    const bool vec = dk % 4 == 0 && dv % 4 == 0 && (io & (bf16 ? 7 : 15)) == 0 &&
                     (((uintptr_t)S0 | (uintptr_t)e) & 15) == 0;
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
