// verify_wide.hip -- packed-tree verification of one Mamba2/SSD layer for wide
// trees (65..256 nodes), bf16 inputs, head_dim 64, d_state 64 or 128.
//
// Method: "STree: Speculative Tree Decoding for Hybrid State Space Models"
// (atlas.scime.ai summary, section "Approach"): per (item b, head h)
//   y_i = exp(cum_i) (h0 C_i) + sum_{j on path(i)} G_ij exp(cum_i - cum_j) dt_j x_j + D x_i,
// G = C B^T on ancestor pairs only, cum = L (dt A) along root paths.
//
// Mapping for MI355X (one work-group of NW = 8 or 16 waves per CU, i.e. two or
// four waves per SIMD, up to ~155 KB of LDS):
//  * work-group = (item b, block of HB heads of one group). The tree set-up
//    (validation, depth by pointer jumping, ancestor-pair lists, pair scores
//    G_ij) runs once and serves all HB heads.
//  * wave w owns node tile NW-1-w (16 nodes) and all 64 rows of head_dim; its
//    C operands (exact bf16 B-matrix of the read-out MFMA) stay in registers for
//    every head of the work-group. Nodes are in topological order, so the last
//    tiles hold the deepest nodes and the longest ancestor walks: they go to the
//    first wave of each SIMD, whose LDS reads are served first in the read-out,
//    so their walks start earliest.
//  * per head, double buffered (head h+1 streams in while head h computes):
//    x (T x 64 bf16) goes straight from HBM to LDS (global_load_lds_dwordx4,
//    whole 128-byte rows); h0 (64 x N fp32) is read once into registers and
//    split once per work-group into bf16 high and low planes in LDS. Tiles are
//    stored with an XOR swizzle of their 16-byte chunks so that the operand
//    and ancestor-row reads below spread over the LDS banks.
//  * read-out (h0 C^T) on 16x16x32 bf16 MFMA (hi and lo planes). The A-operand
//    rows are permuted so that lane (r, q) owns 16 contiguous head_dim columns
//    16q..16q+15 of node 16w + r: ancestor rows of x are two 16-byte LDS reads
//    and y leaves as two 16-byte stores.
//  * the sparse intra-tree term is summed over each node's ancestor-pair list
//    (D x_i joins the node's own term); exp is evaluated on ancestor pairs only
//    and the decay is summed along the path (no cancellation). Two ancestors
//    are taken at a time: their x rows are interleaved into bf16 pairs and
//    dotted (v_dot2_f32_bf16, fp32 accumulate) with the two weights. The masked
//    decay weights are rounded once to bf16, except those of the node's own
//    row (which carries D) and its parent, which keep a bf16 residual as well
//    (about 16 significant bits).
//  * set-up loads (C and B tiles, parents, the step sizes of all HB heads)
//    are independent of the tree and leave together; pair scores are formed
//    from LDS with the B tile passing through the second x buffer.
#include "launch.hpp"
#include "verify_common.hpp"

namespace tsv {

constexpr int kWideMaxPairs = 2048;
// heads one work-group handles at most: the step sizes of all of them are
// staged once, at set-up, as a bf16 [head][node] table in LDS
constexpr int kWideMaxHeads = 20;

template <int NW, int KS>
struct WideCfg {
    static constexpr int NT = NW * kWave;  // threads per work-group
    static constexpr int N = 32 * KS;
    static constexpr int TPM = 16 * NW;    // nodes covered: one 16-node tile per wave
    static constexpr int CPR = N / 8;      // 16-byte bf16 chunks per row of an h0 plane / of C
    static constexpr int HL_BYTES = kHeadDim * N * 2;  // one bf16 plane (hi or lo) of h0
    static constexpr int X_BYTES = TPM * kHeadDim * 2;  // x tile, 128-byte rows
    static constexpr int H0_F4 = kHeadDim * N / 4 / NT; // float4 of h0 per thread
    static constexpr int X_INSTR = TPM * 8 / kWave / NW; // 1 KB async loads per wave
    static_assert(kHeadDim * N / 4 % NT == 0, "h0 tile must split evenly over the threads");
    static_assert(TPM * N * 2 <= 4 * HL_BYTES, "C tile must fit the two h0 buffers");
};

template <int V>
struct BufC {
    static constexpr int value = V;
};

// byte offset of 16-byte chunk c of row r in a tile with `cpr` chunks per row
// (a power of two), chunk index XOR-ed with `key`
__device__ __forceinline__ int swz_off(int r, int c, int cpr, int key) {
    return (r * cpr + (c ^ (key & (cpr - 1)))) * 16;
}
// swizzle key of head_dim row p: the 16 rows one MFMA operand read touches
// (16 (m >> 2) + 4 pt + (m & 3), m = 0..15) get key m, which spreads every
// 16-byte read of the wave over the LDS banks without conflicts (a key that
// is a different bijection of m, such as ((m & 3) << 2) | (m >> 2), leaves
// two-way conflicts)
__device__ __forceinline__ int row_key(int p) { return ((p >> 4) << 2) | (p & 3); }
// swizzle key of x row j: with the row parity it spreads 16 random rows over
// all sixteen 16-byte bank groups
__device__ __forceinline__ int x_key(int j) { return (j >> 1) & 7; }
// head_dim row fed as MFMA A-operand row m of p-tile pt
__device__ __forceinline__ int perm_row(int pt, int m) { return 16 * (m >> 2) + 4 * pt + (m & 3); }

template <int NW, int KS>
__global__ __launch_bounds__(NW * 64, 1) void verify_wide_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const float* __restrict__ D, const float* __restrict__ h0, const int32_t* __restrict__ parent,
    uint16_t* __restrict__ y, int32_t* __restrict__ tree_status, int T, int H, int G, int HB) {
    using Cfg = WideCfg<NW, KS>;
    constexpr int NT = Cfg::NT;
    constexpr int N = Cfg::N;
    constexpr int TPM = Cfg::TPM;
    constexpr int CPR = Cfg::CPR;
    constexpr int MAXP = kWideMaxPairs;

    __shared__ __attribute__((aligned(16))) unsigned char s_hl[2][2][Cfg::HL_BYTES];  // [buf][hi,lo]
    // two distinct arrays (not one indexed by a runtime buffer number) so the
    // compiler can tell that reads of one x buffer never alias the asynchronous
    // loads into the other, and does not wait for the prefetch before them
    __shared__ __attribute__((aligned(16))) unsigned char s_x0[Cfg::X_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char s_x1[Cfg::X_BYTES];
    // dt of every head of the work-group, bf16 [head][node]: one coalesced pass
    // at set-up (a per-head read would touch one cache sector per node per head)
    __shared__ uint16_t s_dth[kWideMaxHeads * TPM];
    __shared__ int s_par[kMaxNodes];
    __shared__ int s_dep[kMaxNodes];
    __shared__ int s_off[kMaxNodes];
    __shared__ int s_scratch[kMaxNodes];
    __shared__ int s_scan[NW];
    __shared__ uint16_t s_pair[MAXP];  // node i in the low byte, ancestor j in the high byte
    __shared__ float s_G[MAXP];

    const int nblk = H / HB;
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int b = blk / nblk;
    const int h_first = (blk % nblk) * HB;
    const int g = h_first / (H / G);
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int r16 = lane & 15;
    const int q = lane >> 4;
    const int tile = NW - 1 - w;  // deepest tiles on the first wave of each SIMD
    const int i = 16 * tile + r16;  // this lane's node
    const size_t bc_row0 = ((size_t)b * T) * G + g;

    // ---- per-head staging
    // x rows of head h straight into LDS buffer `buf` (asynchronous, swizzled)
    auto stage_x = [&](int h, auto bufc) {
        unsigned char* xbase = decltype(bufc)::value == 0 ? s_x0 : s_x1;
#pragma unroll
        for (int m = 0; m < Cfg::X_INSTR; ++m) {
            const int blk = w * Cfg::X_INSTR + m;  // 1 KB block of the tile
            const int pos = blk * kWave + lane;     // 16-byte chunk position in LDS
            const int r = pos >> 3, slot = pos & 7;
            if (r < T)
                __builtin_amdgcn_global_load_lds(
                    (const void*)(x + (((size_t)b * T + r) * H + h) * kHeadDim + 8 * (slot ^ x_key(r))),
                    (__attribute__((address_space(3))) void*)(xbase + blk * 1024), 16, 0, 0);
        }
    };
    // h0 of head h into registers (consecutive threads, consecutive float4)
    float4 hreg[Cfg::H0_F4];
    auto prefetch = [&](int h) {
        const float4* src = (const float4*)(h0 + ((size_t)b * H + h) * kHeadDim * N);
#pragma unroll
        for (int m = 0; m < Cfg::H0_F4; ++m) hreg[m] = src[tid + NT * m];
    };
    // split the registers into bf16 hi / lo planes of buffer `buf`
    auto stage_h0 = [&](int buf) {
        unsigned char* hib = s_hl[buf][0];
        unsigned char* lob = s_hl[buf][1];
#pragma unroll
        for (int m = 0; m < Cfg::H0_F4; ++m) {
            const int gi = tid + NT * m;  // float4 index in the 64 x N tile
            const int p = gi / (N / 4), c4 = gi % (N / 4);
            const int off = swz_off(p, c4 >> 1, CPR, row_key(p)) + 8 * (c4 & 1);
            const float4 v = hreg[m];
            const uint32_t h01 = pack_bf16x2(v.x, v.y), h23 = pack_bf16x2(v.z, v.w);
            const uint32_t l01 = pack_bf16x2(v.x - lo_bf16(h01), v.y - hi_bf16(h01));
            const uint32_t l23 = pack_bf16x2(v.z - lo_bf16(h23), v.w - hi_bf16(h23));
            *(uint2*)(hib + off) = make_uint2(h01, h23);
            *(uint2*)(lob + off) = make_uint2(l01, l23);
        }
    };

    // ---------------------------------------------------------------- set-up
    // The set-up loads leave together: the parents first, then the item's C
    // and B tiles (chunk c = tid + NT m is row c / CPR, chunk column c % CPR)
    // and the step sizes of all HB heads, all into registers; head 0 follows
    // the tree check. Vector memory operations complete in order and every
    // set-up barrier is LDS-only (a __syncthreads would wait for every load in
    // flight), so the tree check waits for the parents only, the pair scores
    // for the B and C tiles only, and the tree work overlaps the rest of the
    // traffic. (No asynchronous LDS load is in flight during the set-up: with
    // one outstanding, the compiler waits for every load at each register use.)
    const int par_i = load_parent(parent + (size_t)b * T, T);
    constexpr int BC_PT = TPM * CPR / NT;                       // tile chunks per thread
    constexpr int DT_PT = (kWideMaxHeads * TPM + NT - 1) / NT;  // step sizes per thread
    uint4 ct[BC_PT], bt[BC_PT];
    uint32_t dtr[DT_PT];
    // (loads are unconditional, from clamped rows, so that the compiler can
    // count the loads still in flight at each later wait; rows past T are zeroed)
#pragma unroll
    for (int m = 0; m < BC_PT; ++m) {
        const int c = tid + NT * m, r = c / CPR, ch = c % CPR;
        const size_t off = (bc_row0 + (size_t)min(r, T - 1) * G) * N + 8 * ch;
        ct[m] = *(const uint4*)(Cm + off);
        bt[m] = *(const uint4*)(Bm + off);
    }
#pragma unroll
    for (int m = 0; m < DT_PT; ++m) {
        const int e = min(tid + NT * m, T * HB - 1);
        const int n = e / HB, hh = e - n * HB;  // consecutive threads: consecutive heads of node n
        dtr[m] = dt[((size_t)b * T + n) * H + h_first + hh];
    }
    const int st = check_tree_lds<NT>(par_i, T, s_par, s_scan);
    if (h_first == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st) return;
    // head 0's h0 and x (16-byte chunk c = tid + NT m is row c / 8, chunk c % 8)
    // only now: issued with the set-up loads, they queue ahead of the parents
    // and tiles of other compute units and delay every set-up step
    prefetch(h_first);
    constexpr int X0_PT = TPM * 8 / NT;
    uint4 x0r[X0_PT];
#pragma unroll
    for (int m = 0; m < X0_PT; ++m) {
        const int c = tid + NT * m, r = min(c >> 3, T - 1);
        x0r[m] = gload((const uint4*)(x + (((size_t)b * T + r) * H + h_first) * kHeadDim + 8 * (c & 7)));
    }
    const int total_pairs = build_pairs<NT>(s_par, T, s_dep, s_off, s_scratch, s_scan, s_pair, MAXP);
    const bool cached = total_pairs <= MAXP;
    // C tile (TPM x N bf16, rows swizzled) in the h0 buffers, which are still free
    unsigned char* cbase = &s_hl[0][0][0];
#pragma unroll
    for (int m = 0; m < BC_PT; ++m) {
        const int c = tid + NT * m, r = c / CPR, ch = c % CPR;
        if (r >= T) ct[m] = bt[m] = make_uint4(0, 0, 0, 0);
        *(uint4*)(cbase + swz_off(r, ch, CPR, r)) = ct[m];
    }
#pragma unroll
    for (int m = 0; m < DT_PT; ++m) {
        const int e = tid + NT * m;
        const int n = e / HB, hh = e - n * HB;
        if (e < T * HB) s_dth[hh * TPM + n] = (uint16_t)dtr[m];
    }
    // pair scores G_ij = C_i . B_j from LDS: the B tile passes through x buffer 1
    // (free until head 1 is staged) 64 columns at a time
    constexpr int PPT = MAXP / NT;  // pairs per thread
    float gacc[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) gacc[k] = 0.f;
#pragma unroll
    for (int pass = 0; pass < N / 64; ++pass) {
#pragma unroll
        for (int m = 0; m < BC_PT; ++m) {
            const int c = tid + NT * m, r = c / CPR, ch = c % CPR;
            if ((ch >> 3) == pass) *(uint4*)(s_x1 + swz_off(r, ch & 7, 8, r)) = bt[m];
        }
        lds_barrier();  // pass columns of B (and, first time, the C tile and pair lists) visible
        if (cached) {
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                const int pq = tid + NT * k;
                if (pq < total_pairs) {
                    const int pr = s_pair[pq];
                    const int pi = pr & 255, pj = pr >> 8;
                    float g0 = 0.f, g1 = 0.f;
#pragma unroll
                    for (int cc = 0; cc < 8; cc += 2) {
                        g0 = dot8_bf16(*(const uint4*)(cbase + swz_off(pi, 8 * pass + cc, CPR, pi)),
                                       *(const uint4*)(s_x1 + swz_off(pj, cc, 8, pj)), g0);
                        g1 = dot8_bf16(*(const uint4*)(cbase + swz_off(pi, 8 * pass + cc + 1, CPR, pi)),
                                       *(const uint4*)(s_x1 + swz_off(pj, cc + 1, 8, pj)), g1);
                    }
                    gacc[k] += g0 + g1;
                }
            }
        }
        lds_barrier();  // B columns consumed
    }
    if (cached) {
#pragma unroll
        for (int k = 0; k < PPT; ++k)
            if (tid + NT * k < total_pairs) s_G[tid + NT * k] = gacc[k];
    }
    bf16x8 creg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) creg[ks] = *(const bf16x8*)(cbase + swz_off(i, 4 * ks + q, CPR, i));
    const int my_base = (i < T) ? s_off[i] : 0;
    const int my_cnt = (i < T) ? s_dep[i] + 1 : 0;
    lds_barrier();  // C tile consumed: the h0 buffers are free
    stage_h0(0);
#pragma unroll
    for (int m = 0; m < X0_PT; ++m) {
        const int c = tid + NT * m, r = c >> 3;
        if (r < T) *(uint4*)(s_x0 + swz_off(r, c & 7, 8, x_key(r))) = x0r[m];
    }
    lds_barrier();

    // ---------------------------------------------------------------- heads
    const bool tile_live = 16 * tile < T;
    auto head = [&](int hh, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const int h = h_first + hh;
        const bool more = hh + 1 < HB;
        if (more) {
            stage_x(h + 1, BufC<buf ^ 1>{});
            prefetch(h + 1);
        }
        uint32_t o[8];
        if (tile_live) {
            const unsigned char* hib = s_hl[buf][0];
            const unsigned char* lob = s_hl[buf][1];
            const unsigned char* sx = buf == 0 ? s_x0 : s_x1;
            const uint16_t* sdt = s_dth + hh * TPM;

            // read-out: acc[pt] holds (h0 C^T) rows p = 16q + 4pt + r, column i
            f32x4 acc[4];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int p = perm_row(pt, r16);
                    const int off = swz_off(p, 4 * ks + q, CPR, row_key(p));
                    acc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(hib + off), creg[ks], acc[pt], 0, 0, 0);
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int p = perm_row(pt, r16);
                    const int off = swz_off(p, 4 * ks + q, CPR, row_key(p));
                    acc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(lob + off), creg[ks], acc[pt], 0, 0, 0);
                }
            }

            // intra-tree term + D x_i over node i's ancestor list, columns 16q .. 16q+15,
            // two ancestors at a time: their x rows are interleaved into bf16 pairs and
            // multiplied by the two weights (v_dot2_f32_bf16, fp32 accumulate)
            const float Ah = A[h];
            const float Dh = D[h];
            float ta[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) ta[e] = 0.f;
            // LO: also multiply by the bf16 residuals of the weights (about 16
            // significant bits in all); used for the node's own row, which carries
            // D, and its parent
            auto add_rows = [&](int j0, float w0, int j1, float w1, auto loc) {
                constexpr bool LO = decltype(loc)::value != 0;
                const int a0 = swz_off(j0, 2 * q, 8, x_key(j0));
                const int a1 = swz_off(j1, 2 * q, 8, x_key(j1));
                const uint4 p0 = *(const uint4*)(sx + a0), q0 = *(const uint4*)(sx + (a0 ^ 16));
                const uint4 p1 = *(const uint4*)(sx + a1), q1 = *(const uint4*)(sx + (a1 ^ 16));
                const uint32_t u0[8] = {p0.x, p0.y, p0.z, p0.w, q0.x, q0.y, q0.z, q0.w};
                const uint32_t u1[8] = {p1.x, p1.y, p1.z, p1.w, q1.x, q1.y, q1.z, q1.w};
                const uint32_t whi = pack_bf16x2(w0, w1);
                const bf16x2 wh = __builtin_bit_cast(bf16x2, whi);
                const bf16x2 wl = __builtin_bit_cast(bf16x2, pack_bf16x2(w0 - lo_bf16(whi), w1 - hi_bf16(whi)));
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bf16x2 xl = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(u1[e], u0[e], 0x05040100u));
                    const bf16x2 xh = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(u1[e], u0[e], 0x07060302u));
                    ta[2 * e] = __builtin_amdgcn_fdot2_f32_bf16(xl, wh, ta[2 * e], false);
                    ta[2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(xh, wh, ta[2 * e + 1], false);
                    if (LO) {
                        ta[2 * e] = __builtin_amdgcn_fdot2_f32_bf16(xl, wl, ta[2 * e], false);
                        ta[2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(xh, wl, ta[2 * e + 1], false);
                    }
                }
            };
            float s = 0.f;  // sum of dt*A over the path nodes from i up to (excluding) j
            if (i < T) {
                if (cached) {
                    // entries k and k+1 of the list; entry 0 is the node itself with
                    // weight G_ii dt_i + D. The first two rows take the weights to
                    // about 16 bits, the older ancestors to bf16.
                    // The list entries of the next pair are read while the
                    // current pair's rows are in flight, so each step waits for
                    // one LDS round trip rather than two.
                    const int last = my_cnt - 1;
                    int pr0 = s_pair[my_base], pr1 = s_pair[my_base + min(1, last)];
                    float g0 = s_G[my_base], g1 = s_G[my_base + min(1, last)];
                    auto pair_step = [&](int k, auto loc) {
                        const int kn0 = min(k + 2, last), kn1 = min(k + 3, last);
                        const int npr0 = s_pair[my_base + kn0], npr1 = s_pair[my_base + kn1];
                        const float ng0 = s_G[my_base + kn0], ng1 = s_G[my_base + kn1];
                        const int j0 = pr0 >> 8;
                        const float dj0 = bf16_bits_to_f32(sdt[j0]);
                        const float w0 = g0 * __expf(s) * dj0 + (k == 0 ? Dh : 0.f);
                        s += dj0 * Ah;
                        int j1 = j0;
                        float w1 = 0.f;
                        if (k + 1 < my_cnt) {
                            j1 = pr1 >> 8;
                            const float dj1 = bf16_bits_to_f32(sdt[j1]);
                            w1 = g1 * __expf(s) * dj1;
                            s += dj1 * Ah;
                        }
                        add_rows(j0, w0, j1, w1, loc);
                        pr0 = npr0;
                        pr1 = npr1;
                        g0 = ng0;
                        g1 = ng1;
                    };
                    pair_step(0, BufC<1>{});
                    for (int k = 2; k < my_cnt; k += 2) pair_step(k, BufC<0>{});
                } else {
                    // pair list too long for LDS (very deep trees): chase parents and
                    // score each pair from the B and C rows in memory
                    const uint16_t* Ci = Cm + (bc_row0 + (size_t)i * G) * N;
                    for (int j = i; j >= 0; j = s_par[j]) {
                        const float dj = bf16_bits_to_f32(sdt[j]);
                        const float gij = dot_rows_lean<N>(Ci, Bm + (bc_row0 + (size_t)j * G) * N);
                        add_rows(j, gij * __expf(s) * dj + (j == i ? Dh : 0.f), j, 0.f, BufC<1>{});
                        s += dj * Ah;
                    }
                }
            }
            const float sc = __expf(s);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int pt = e >> 1, r = 2 * (e & 1);  // columns 4pt + r, 4pt + r + 1
                o[e] = pack_bf16x2(acc[pt][r] * sc + ta[2 * e], acc[pt][r + 1] * sc + ta[2 * e + 1]);
            }
        }
        // Stage head h+1 before storing y: on gfx9 the wait also counts stores, so
        // stores issued first would be waited for here. The wait sits outside every
        // branch so that no path reaches the barrier with an asynchronous LDS load
        // still in flight (the compiler would otherwise wait for the y stores too).
        __builtin_amdgcn_s_waitcnt(0);  // head h+1: this thread's h0 and x chunks landed
        if (more) stage_h0(buf ^ 1);
        if (tile_live && i < T) {
            uint4* dst = (uint4*)(y + (((size_t)b * T + i) * H + h) * kHeadDim + 16 * q);
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
        // head h+1 staged (its asynchronous x loads were waited for above); buffer
        // buf free for head h+2. The y stores of head h stay in flight.
        lds_barrier();
    };
    for (int hh = 0; hh < HB; hh += 2) {
        head(hh, BufC<0>{});
        if (hh + 1 < HB) head(hh + 1, BufC<1>{});
    }
}

template <int NW, int KS>
static const void* wide_kernel() { return (const void*)verify_wide_kernel<NW, KS>; }

static int wide_waves(int T) { return T <= 128 ? 8 : 16; }

static const void* pick_wide(int T, int N) {
    if (N == 64) return wide_waves(T) == 8 ? wide_kernel<8, 2>() : wide_kernel<16, 2>();
    return wide_waves(T) == 8 ? wide_kernel<8, 4>() : wide_kernel<16, 4>();
}

hipError_t launch_verify_wide(const VerifyArgs& a, int HB, hipStream_t stream) {
    // heads per work-group: the largest divisor of the requested count that the
    // LDS step-size table holds (results do not depend on it)
    int hb = 1;
    for (int d = 1; d <= kWideMaxHeads && d <= HB; ++d)
        if (HB % d == 0) hb = d;
    HB = hb;
    const void* k = pick_wide(a.T, a.N);
    dim3 grid((unsigned)(a.batch * (a.H / HB)));
    void* args[] = {(void*)&a.x, (void*)&a.dt, (void*)&a.A, (void*)&a.B, (void*)&a.C, (void*)&a.D,
                    (void*)&a.h0, (void*)&a.parent, (void*)&a.y, (void*)&a.tree_status,
                    (void*)&a.T, (void*)&a.H, (void*)&a.G, (void*)&HB};
    return hipLaunchKernel(k, grid, dim3(wide_waves(a.T) * kWave), args, 0, stream);
}

}  // namespace tsv
