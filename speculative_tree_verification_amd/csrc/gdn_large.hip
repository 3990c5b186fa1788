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
// e is written only if the caller asks for it.
//
// One work-group of 16 waves per (item, head); wave w owns nodes [16 w, 16 w + 16):
//  1. tree check, depth and every node's ancestor list (itself first, then up
//     to the root) in LDS; a tree with more than kGdnLargePairs
//     ancestor-or-self pairs is reported with status 8 and left untouched.
//     S0 is staged in LDS as bf16 high and low parts, in the order the MFMA B
//     operand reads it (one linear 1 KB read per wave and step), once the
//     pair scores are done with the same LDS.
//  2. pair scores of the wave's nodes from the k and q columns its lanes
//     hold as MFMA A operands and the same columns of each ancestor's k row,
//     from LDS, where every wave puts its nodes' rows (fp32 rows half of the
//     columns at a time), so k is read from memory once;
//  3. Q S0^T and K S0^T for the wave's 16 nodes on MFMA (three-term bf16
//     splits, fp32 accumulation; two terms for bf16 inputs, whose low parts
//     are zero; bf16 v already on its way), and r in registers. The column order of the product tiles
//     gives each lane four consecutive value rows twice, so v, r, e and o
//     move as 16-byte vectors;
//  4. M row by row, one thread a row, from M (I + A) = I:
//        M_ij = -sum_{x from i down to j, x != j} M_ix A_xj   (M_ii = 1),
//     each entry from the row's entries before it (no barrier per depth
//     level); then N_ij = sum_{x from i down to j} W_ix M_xj, all at once;
//  5. e_i = sum_j M_ij r_j and o_i = exp(G_i) (S0 q_i) + sum_j N_ij r_j over the
//     root path of i, one half of the value rows at a time: that half of r
//     (64 floats per node, 64 KB) sits in LDS where the S0 planes were, so r
//     never goes to memory.
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

// The lane's share of a node row as the 16 x 32 A operand of the products:
// lane (l16, q4) holds columns 32 ks + 8 q4 .. + 7 for every step ks (zero
// past dk or past the tree); fp32 rows as floats, bf16 rows as their bits
template <typename TIO>
struct ARow;
template <>
struct ARow<float> {
    float4 v[2 * kLKS];
};
template <>
struct ARow<uint16_t> {
    uint4 v[kLKS];
};

// With VEC (rows of a multiple of four elements) the loads are unconditional,
// from columns clamped into the row, and the values past dk or past the tree
// are zeroed afterwards: the compiler can then count how many of them are
// still in flight at a wait (branches around loads make it wait for all).
template <typename TIO, bool VEC>
__device__ __forceinline__ void load_a(const TIO* __restrict__ row, bool live, int q4, int dk, ARow<TIO>& a) {
#pragma unroll
    for (int ks = 0; ks < kLKS; ++ks) {
        const int c = 32 * ks + 8 * q4;
        const bool in0 = live && c < dk, in1 = live && c + 4 < dk;
        if constexpr (sizeof(TIO) == 4) {
            if (VEC) {
                const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                const float4 x0 = ld4<true>(row + min(c, dk - 4), 4), x1 = ld4<true>(row + min(c + 4, dk - 4), 4);
                a.v[2 * ks] = in0 ? x0 : z;
                a.v[2 * ks + 1] = in1 ? x1 : z;
            } else {
                a.v[2 * ks] = a.v[2 * ks + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (in0) a.v[2 * ks] = ld4<false>(row + c, dk - c);
                if (in1) a.v[2 * ks + 1] = ld4<false>(row + c + 4, dk - c - 4);
            }
        } else {
            a.v[ks] = make_uint4(0u, 0u, 0u, 0u);
            if (VEC) {
                const uint2 x0 = gload((const uint2*)(row + min(c, dk - 4)));
                const uint2 x1 = gload((const uint2*)(row + min(c + 4, dk - 4)));
                a.v[ks] = make_uint4(in0 ? x0.x : 0u, in0 ? x0.y : 0u, in1 ? x1.x : 0u, in1 ? x1.y : 0u);
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    if (live && c + t < dk) w[t >> 1] |= (uint32_t)gload(row + c + t) << (16 * (t & 1));
                a.v[ks] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }
}

// bf16 high and low parts of step ks (bf16 rows: the bits, and no low part)
template <typename TIO>
__device__ __forceinline__ void a_parts(const ARow<TIO>& a, int ks, bf16x8& hi, bf16x8& lo) {
    if constexpr (sizeof(TIO) == 4) {
        split_hi_lo(a.v[2 * ks], a.v[2 * ks + 1], hi, lo);
    } else {
        hi = __builtin_bit_cast(bf16x8, a.v[ks]);
        lo = hi;  // unused
    }
}

// partial dot products of two rows over the lane's columns (fp32 arithmetic;
// bf16 products are exact in it)
template <typename TIO>
__device__ __forceinline__ float a_dot(const ARow<TIO>& a, const ARow<TIO>& b) {
    float s = 0.f;
    if constexpr (sizeof(TIO) == 4) {
#pragma unroll
        for (int u = 0; u < 2 * kLKS; ++u)
            s += (a.v[u].x * b.v[u].x + a.v[u].y * b.v[u].y) + (a.v[u].z * b.v[u].z + a.v[u].w * b.v[u].w);
    } else {
#pragma unroll
        for (int u = 0; u < kLKS; ++u) s = dot8_bf16(a.v[u], b.v[u], s);
    }
    return s;
}

// X S0^T for the wave's 16 nodes: acc[nb] holds (node 16 w + 4 q4 + r, value
// row vrow(nb, l16)) in element r
template <typename TIO>
__device__ __forceinline__ void s0_product(const ARow<TIO>& a, const bf16x8* __restrict__ s_S0, int lane, int dk,
                                           int dv, f32x4* acc) {
    constexpr bool BF = sizeof(TIO) == 2;
#pragma unroll
    for (int nb = 0; nb < kLNB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kLKS; ++ks) {
        if (32 * ks >= dk) break;
        bf16x8 ah, al;
        a_parts<TIO>(a, ks, ah, al);
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
    const float gi = g[row0 + (size_t)min(tid, T - 1) * H];
    const float bi = beta[row0 + (size_t)min(tid, T - 1) * H];
    // S0 and the wave's k and q rows leave with the parents. The loads are
    // unconditional, from clamped addresses where the shapes allow, so that
    // the tree check waits for the parents only (branches around loads make
    // the compiler wait for all of them); the parents still come back behind
    // much of every work-group's burst. Issuing the burst after the check
    // instead moved the same wait into the pair lists (a wave stalls on
    // issuing loads whose queue is full): no faster.
    float4 s0v[4];  // B-operand entries tid and tid + NT: S0[vrow(nb, l16')][32 ks + 8 q4' .. + 7]
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int x = tid + NT * u, ln = x & (kWave - 1), ks = (x / kWave) % kLKS, nb = x / (kWave * kLKS);
        const int p = vrow(nb, ln & 15), c = 32 * ks + 8 * (ln >> 4);
        const bool in0 = p < dv && c < dk, in1 = p < dv && c + 4 < dk;
        if (VEC) {  // zeroed past the matrix when staged
            const float* src = S0h + (size_t)min(p, dv - 1) * dk;
            s0v[2 * u] = ld4<true>(src + min(c, dk - 4), 4);
            s0v[2 * u + 1] = ld4<true>(src + min(c + 4, dk - 4), 4);
        } else {
            s0v[2 * u] = s0v[2 * u + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (in0) s0v[2 * u] = ld4<false>(S0h + (size_t)p * dk + c, dk - c);
            if (in1) s0v[2 * u + 1] = ld4<false>(S0h + (size_t)p * dk + c + 4, dk - c - 4);
        }
    }
    const int ia = 16 * w + l16;  // A-operand row of this lane
    const bool alive = rows && ia < T;
    ARow<TIO> ka, qa;
    load_a<TIO, VEC>(k + (row0 + (size_t)min(ia, T - 1) * H) * dk, alive, q4, dk, ka);
    load_a<TIO, VEC>(q + (row0 + (size_t)min(ia, T - 1) * H) * dk, alive, q4, dk, qa);
    const int i4 = 16 * w + 4 * q4;  // nodes i4 .. i4 + 3 of this lane's accumulators

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
    }
    constexpr bool BF = sizeof(TIO) == 2;
    lds_barrier();

    // partial log decays along each list, exp(G_i), list starts, M_ii
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
    }
    lds_barrier();

    // ---- 2. pair scores: lane (l16, q4) dots the columns it holds of k_i and
    // q_i (i = ia, its A-operand row) with the same columns of each
    // ancestor's k_j, and the four lanes of node i add up. Every wave first
    // puts its nodes' k rows into LDS, where the S0 planes go later (256
    // bytes a node: bf16 rows whole, fp32 rows 64 columns a pass, the first
    // pass's partial sums parked in W and in M's strict-ancestor entries,
    // which the solve writes later), so k is read from memory once. A row's
    // 16-byte chunks are XOR-swizzled with the node index: the 16 lanes that
    // read the same column of 16 different rows then hit different banks.
    f32x4 qs[kLNB];
    float4 rr[8];  // r at the accumulator positions: node i4 + r, value rows 64 hf + 4 l16 .. + 3
    const int cnt = alive ? s_dep[ia] + 1 : 0, base = alive ? s_off[ia] : 0;
    constexpr int PASSES = BF ? 1 : 2;
    constexpr int KSP = kLKS / PASSES;  // contraction steps per pass
    constexpr int EPC = 16 / sizeof(TIO);  // elements per 16-byte chunk
    TIO* const s_k = (TIO*)s_S0;           // [node][16 chunks]
    // element offset of chunk ch of node n's row
    auto kchunk = [&](int n, int ch) { return (n * 16 + (ch ^ (n & 15))) * EPC; };
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        if (ps > 0) lds_barrier();  // the first pass's reads are done
        if (alive) {
#pragma unroll
            for (int t = 0; t < KSP; ++t) {
                const int ks = ps * KSP + t;
                if constexpr (BF) {
                    *(uint4*)&s_k[kchunk(ia, 4 * t + q4)] = ka.v[ks];
                } else {
                    *(float4*)&s_k[kchunk(ia, 8 * t + 2 * q4)] = ka.v[2 * ks];
                    *(float4*)&s_k[kchunk(ia, 8 * t + 2 * q4 + 1)] = ka.v[2 * ks + 1];
                }
            }
        }
        lds_barrier();
        if (rows) {
            for (int m = 0; m < cnt; ++m) {
                const int j = s_pair[base + m] >> 8;
                float kk = 0.f, qk = 0.f;
#pragma unroll
                for (int t = 0; t < KSP; ++t) {
                    const int ks = ps * KSP + t;
                    if constexpr (BF) {
                        const uint4 kj = *(const uint4*)&s_k[kchunk(j, 4 * t + q4)];
                        kk = dot8_bf16(ka.v[ks], kj, kk);
                        qk = dot8_bf16(qa.v[ks], kj, qk);
                    } else {
                        const float4 k0 = *(const float4*)&s_k[kchunk(j, 8 * t + 2 * q4)];
                        const float4 k1 = *(const float4*)&s_k[kchunk(j, 8 * t + 2 * q4 + 1)];
                        const float4 a0 = ka.v[2 * ks], a1 = ka.v[2 * ks + 1];
                        const float4 q0 = qa.v[2 * ks], q1 = qa.v[2 * ks + 1];
                        kk += (a0.x * k0.x + a0.y * k0.y) + (a0.z * k0.z + a0.w * k0.w) +
                              ((a1.x * k1.x + a1.y * k1.y) + (a1.z * k1.z + a1.w * k1.w));
                        qk += (q0.x * k0.x + q0.y * k0.y) + (q0.z * k0.z + q0.w * k0.w) +
                              ((q1.x * k1.x + q1.y * k1.y) + (q1.z * k1.z + q1.w * k1.w));
                    }
                }
                kk += __shfl_xor(kk, 16, kWave);
                qk += __shfl_xor(qk, 16, kWave);
                kk += __shfl_xor(kk, 32, kWave);
                qk += __shfl_xor(qk, 32, kWave);
                if (q4 == 0) {
                    if (ps + 1 < PASSES) {
                        if (m > 0) s_M[base + m] = kk;
                        s_W[base + m] = qk;
                    } else {
                        if (ps > 0) {
                            kk += m > 0 ? s_M[base + m] : 0.f;
                            qk += s_W[base + m];
                        }
                        const float D = __expf(s_A[base + m]);
                        s_A[base + m] = m > 0 ? s_bt[ia] * D * kk : 0.f;
                        s_W[base + m] = D * qk;
                    }
                }
            }
        }
    }
    // v at the accumulator positions (node i4 + r, value rows 64 hf + 4 l16 .. + 3;
    // VEC: unconditional, from clamped addresses, zeroed past the matrix).
    // bf16 rows (whole 8-byte vectors) leave now, to arrive while S0 is
    // staged and the products run; fp32 rows only after the products (holding
    // them through the products would spill)
    auto load_v = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int i = i4 + r, p0 = 64 * hf + 4 * l16;
                if (VEC) {
                    const float4 x = ld4io<TIO, true>(v + (row0 + (size_t)min(i, T - 1) * H) * dv + min(p0, dv - 4), 4);
                    rr[2 * r + hf] = i < T && p0 < dv ? x : make_float4(0.f, 0.f, 0.f, 0.f);
                } else {
                    rr[2 * r + hf] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (i < T && p0 < dv) rr[2 * r + hf] = ld4io<TIO, false>(v + (row0 + (size_t)i * H) * dv + p0, dv - p0);
                }
            }
    };
    constexpr bool EARLY_V = BF && VEC;
    if constexpr (EARLY_V) {
        if (rows) load_v();
        __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();  // every k row has been read: the S0 planes go in
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (VEC) {
            const int x = tid + NT * u, ln = x & (kWave - 1), ks = (x / kWave) % kLKS, nb = x / (kWave * kLKS);
            const int p = vrow(nb, ln & 15), c = 32 * ks + 8 * (ln >> 4);
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            if (!(p < dv && c < dk)) s0v[2 * u] = z;
            if (!(p < dv && c + 4 < dk)) s0v[2 * u + 1] = z;
        }
        bf16x8 hi, lo;
        split_hi_lo(s0v[2 * u], s0v[2 * u + 1], hi, lo);
        s_S0[tid + NT * u] = hi;
        s_S0[kS0Ent + tid + NT * u] = lo;
    }
    lds_barrier();

    if (rows) {
        // ---- 3. Q S0^T (kept), K S0^T, and r = beta (v - exp(G) K S0^T)
        s0_product<TIO>(qa, s_S0, lane, dk, dv, qs);
        f32x4 ks_[kLNB];
        s0_product<TIO>(ka, s_S0, lane, dk, dv, ks_);
        if constexpr (!EARLY_V) {
            __builtin_amdgcn_sched_barrier(0);
            load_v();
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = min(i4 + r, T - 1);
            const float bt = s_bt[i], gm = s_gam[i];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const float4 x = rr[2 * r + hf];
                rr[2 * r + hf] = make_float4(bt * (x.x - gm * ks_[4 * hf][r]), bt * (x.y - gm * ks_[4 * hf + 1][r]),
                                             bt * (x.z - gm * ks_[4 * hf + 2][r]),
                                             bt * (x.w - gm * ks_[4 * hf + 3][r]));
            }
        }
    }
    lds_barrier();  // the pair scores are complete, and no wave reads the S0 planes any more

    // r of value rows 0..63 goes where the S0 planes were: a 64-float row per node
    float* const s_r = (float*)s_S0;
    auto stage_r = [&](int hf) {
        if (!rows) return;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (i4 + r < T) *(float4*)&s_r[(i4 + r) * 64 + 4 * l16] = rr[2 * r + hf];
    };
    stage_r(0);

    // ---- 4. M = (I + A)^{-1} row by row, from M (I + A) = I: entry m of node
    // i's list (its ancestor m steps up) follows from the entries before it in
    // the same row, M_{i,m} = -sum_{m' < m} M_{i,m'} A_{x(m'), m - m'}, with
    // x(m') the ancestor m' steps up and M_{i,0} = 1. One thread a row and no
    // barrier between depth levels.
    if (tid < T) {
        const int base = s_off[tid], cnt = s_dep[tid] + 1;
        for (int m = 1; m < cnt; ++m) {
            float acc = 0.f;
            for (int m0 = 0; m0 < m; m0 += 4) {
                float mv[4], av[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int mm = min(m0 + u, m - 1);
                    mv[u] = s_M[base + mm];
                    av[u] = s_A[s_aof[base + mm] + m - mm];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (m0 + u < m) acc -= mv[u] * av[u];
            }
            s_M[base + m] = acc;
        }
    }
    lds_barrier();
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
    lds_barrier();  // N and the first half of r are complete

    // ---- 5. e = M r and o = exp(G) (Q S0^T) + N r over each root path, one
    // half of the value rows at a time (r from LDS)
    for (int hf = 0; hf < 2; ++hf) {
        if (64 * hf >= dv) break;
        if (hf == 1) {
            lds_barrier();  // every wave is done with the first half
            stage_r(1);
            lds_barrier();
        }
        const int p0 = 64 * hf + 4 * l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i4 + r;
            if (!rows || i >= T) continue;
            const float gm = s_gam[i];
            float4 ea = make_float4(0.f, 0.f, 0.f, 0.f);
            float4 oa = make_float4(gm * qs[4 * hf][r], gm * qs[4 * hf + 1][r], gm * qs[4 * hf + 2][r],
                                    gm * qs[4 * hf + 3][r]);
            const int base = s_off[i], cnt = s_dep[i] + 1;
            for (int m0 = 0; m0 < cnt; m0 += 4) {
                float4 rv[4];
                float mv[4], nv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int mm = min(m0 + u, cnt - 1);
                    rv[u] = *(const float4*)&s_r[(s_pair[base + mm] >> 8) * 64 + 4 * l16];
                    mv[u] = m0 + u < cnt ? s_M[base + mm] : 0.f;
                    nv[u] = m0 + u < cnt ? s_A[base + mm] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ea.x += mv[u] * rv[u].x;
                    ea.y += mv[u] * rv[u].y;
                    ea.z += mv[u] * rv[u].z;
                    ea.w += mv[u] * rv[u].w;
                    oa.x += nv[u] * rv[u].x;
                    oa.y += nv[u] * rv[u].y;
                    oa.z += nv[u] * rv[u].z;
                    oa.w += nv[u] * rv[u].w;
                }
            }
            if (p0 < dv) {
                st4io<TIO, VEC>(o + (row0 + (size_t)i * H) * dv + p0, oa, dv - p0);
                if (e) st4io<float, VEC>(e + (row0 + (size_t)i * H) * dv + p0, ea, dv - p0);
            }
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
