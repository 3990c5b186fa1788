// verify_mfma.hip -- packed-tree verification of one Mamba2/SSD layer, bf16
// inputs, head_dim 64, d_state 64 or 128, trees of up to 64 nodes, on gfx950
// matrix cores (wider trees: verify_wide.hip).
//
// Method: "STree: Speculative Tree Decoding for Hybrid State Space Models"
// (atlas.scime.ai summary, section "Approach"; mlsanity abstract): log decays
// accumulated along ancestor paths of the packed tree (A_tree = L log A) give
// every node's exact per-path output in one pass. Per (item b, head h):
//   y_i = exp(cum_i) h0 C_i                                  (state read-out)
//       + sum_{j on path(i)} G_ij exp(cum_i - cum_j) dt_j x_j  (intra-tree term)
//       + D x_i,                     G = C B^T of the head's group.
//
// Mapping (MI355X: 64-wide waves, 16x16x32 bf16 MFMA, 160 KB LDS):
//  * work-group = (item b, HW heads of one group), 4 HW waves: the four waves
//    of head slot s = w / 4 own head_dim rows 16 (w % 4) .. +15 of that head.
//    Every head of the work-group is computed at the same time; small trees
//    give too little work per head to hide memory latency head after head.
//  * set-up, once per work-group: the tree is validated, and the pair scores
//    G = C B^T of the lower-triangular 16 x 16 node tiles are formed on MFMA
//    (at most ten 16 x 16 tiles for 64 nodes, a few MFMAs per wave) and kept
//    in LDS for all HW heads. No pair list is built: each lane walks its
//    node's root path through the parents in LDS, and the next parent, the
//    step size, the x row and the score of an ancestor are read in one round.
//  * every load leaves at the start, the parents first: no load depends on
//    the tree, and vector memory operations complete in order, so the tree
//    check waits for the parents only while the rest (B and C tiles, step
//    sizes, each wave's 16 x N slice of h0 and its x rows) streams in.
//  * the read-out C h0^T runs on MFMA with h0 split into bf16 high + low
//    halves (about 16 significant bits), one k-step at a time; C is an exact
//    bf16 operand kept in registers.
//  * the intra-tree term is sparse (depth+1 terms per node), so it is summed
//    along each node's root path in fp32 VALU, with exp evaluated only on
//    ancestor pairs and the decay summed along the path (no cancellation).
#include "launch.hpp"
#include "verify_common.hpp"

namespace tsv {

constexpr int kP = kHeadDim;
constexpr int kXStride = 20;        // LDS row stride (uint16) of a wave's 16-column x slice
constexpr int kSmallMaxHeads = 4;   // heads per work-group at most (16 waves)

template <int TI, int HW>
struct MfmaCfg {
    static constexpr int NT = 4 * HW * kWave;  // threads per work-group
    static constexpr int TP = 16 * TI;         // node count padded to whole 16-node tiles
    static constexpr int kXChunks = (2 * TP + kWave - 1) / kWave;
};

// One-head work-groups (HW = 1) are sized for five per compute unit, so that
// the batch-16 layer (1,280 work-groups) is resident in a single round.
template <int TI, int KS, int HW>
__global__ __launch_bounds__(4 * HW * 64) __attribute__((amdgpu_waves_per_eu(HW == 1 ? 5 : 1)))
void verify_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const float* __restrict__ D, const float* __restrict__ h0, const int32_t* __restrict__ parent,
    uint16_t* __restrict__ y, int32_t* __restrict__ tree_status, int T, int H, int G) {
    using Cfg = MfmaCfg<TI, HW>;
    // one-head work-groups read h0 in whole 1 KB runs per instruction and
    // store y as whole rows; wider ones read h0 in MFMA operand order
    constexpr bool LIN = HW == 1;
    constexpr int NT = Cfg::NT;
    constexpr int N = 32 * KS;
    constexpr int TP = Cfg::TP;

    __shared__ int s_par[kMaxNodes];
    // pair scores G_ij = C_i . B_j, fp32 [i][j], lower-triangular 16 x 16 tiles
    __shared__ float s_G[TP * TP];
    __shared__ __attribute__((aligned(16))) uint16_t s_x[4 * HW][TP * kXStride];
    __shared__ uint16_t s_dth[HW * TP];  // dt of the work-group's heads, bf16 [slot][node]
    // B and C rows of the item's group, padded by 16 bytes per row; once the
    // pair scores and the C operands are taken, the same memory stages h0
    // (one-head work-groups: each wave's 16 x N slice, one bf16 plane at a time)
    constexpr int BCS = N + 8;
    constexpr int kStage = LIN ? 4 * 16 * N : 0;
    constexpr int kBC = 2 * TP * BCS > kStage ? 2 * TP * BCS : kStage;
    __shared__ __attribute__((aligned(16))) uint16_t s_BC[kBC];
    uint16_t* const s_Bt = s_BC;
    uint16_t* const s_Ct = s_BC + TP * BCS;
    // y rows of the work-group's head (one-head work-groups), 16 bytes of padding
    // per row, so that y leaves as whole 128-byte rows
    constexpr int kYS = kP + 8;
    __shared__ __attribute__((aligned(16))) uint16_t s_y[LIN ? TP * kYS : 8];

    const int nblk = H / HW;
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int b = blk / nblk;
    const int h_first = (blk % nblk) * HW;
    const int g = h_first / (H / G);
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int wl = w & 3;                                        // head_dim slice of this wave
    const int slot = w >> 2;                                     // head slot of this wave
    const int h = h_first + slot;
    const int r16 = lane & 15;
    const int q = lane >> 4;
    const size_t bc_row0 = ((size_t)b * T) * G + g;  // row (b, node 0, g) of B and C

    // ---------------------------------------------------------------- loads
    // (unconditional, from clamped rows, so that the compiler can count the
    // loads still in flight at each wait; rows past T are zeroed or unused)
    const int par_i = load_parent(parent + (size_t)b * T, T);
    constexpr int CPR = N / 8;
    constexpr int BC_PT = (TP * CPR + NT - 1) / NT;
    constexpr int DT_PT = (HW * TP + NT - 1) / NT;
    uint4 breg[BC_PT], cregt[BC_PT];
#pragma unroll
    for (int m = 0; m < BC_PT; ++m) {
        const int c = tid + NT * m;
        const int r = min(c / CPR, T - 1), ch = c % CPR;
        breg[m] = *(const uint4*)(Bm + (bc_row0 + (size_t)r * G) * N + 8 * ch);
        cregt[m] = *(const uint4*)(Cm + (bc_row0 + (size_t)r * G) * N + 8 * ch);
    }
    uint32_t dtr[DT_PT];
#pragma unroll
    for (int m = 0; m < DT_PT; ++m) {
        const int e = min(tid + NT * m, T * HW - 1);
        const int n = e / HW, hh = e - n * HW;  // consecutive threads: consecutive heads of node n
        dtr[m] = dt[((size_t)b * T + n) * H + h_first + hh];
    }
    // this wave's 16 x N slice of h0 (rows 16 wl .. 16 wl + 15) and its 16
    // columns of x. One-head work-groups read the slice as 2 KS consecutive
    // 1 KB runs (float4 m of lane l is element 4 (l + 64 m) of the slice),
    // streamed past the caches: this access pattern alone took the launch's
    // memory skeleton (loads and stores, no arithmetic) from 15.0 to 13.8 us,
    // 12.4 us with the nontemporal hint, at batch 16 x 31 nodes x 80 heads.
    // The slice reaches MFMA operand order through LDS after the set-up.
    float4 hr[KS][2];
    if (LIN) {
        const float4* hblk = (const float4*)(h0 + (((size_t)b * H + h) * kP + 16 * wl) * N);
#pragma unroll
        for (int m = 0; m < 2 * KS; ++m) hr[m >> 1][m & 1] = gload_nt(hblk + lane + kWave * m);
    } else {
        const float* hrow = h0 + (((size_t)b * H + h) * kP + 16 * wl + r16) * N + 8 * q;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            hr[ks][0] = *(const float4*)(hrow + 32 * ks);
            hr[ks][1] = *(const float4*)(hrow + 32 * ks + 4);
        }
    }
    uint4 xr[Cfg::kXChunks];
#pragma unroll
    for (int m = 0; m < Cfg::kXChunks; ++m) {
        const int c = lane + kWave * m;
        const int row = min(c >> 1, T - 1), half = c & 1;  // rows past T are not staged
        xr[m] = *(const uint4*)(x + (((size_t)b * T + row) * H + h) * kP + 16 * wl + 8 * half);
    }

    // ---------------------------------------------------------------- set-up
    const int st = check_tree(par_i, T, s_par);
    if (h_first == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st) return;
#pragma unroll
    for (int m = 0; m < BC_PT; ++m) {
        const int c = tid + NT * m;
        const int r = c / CPR, ch = c % CPR;
        if (r < TP) {
            const bool live = r < T;
            *(uint4*)(s_Bt + r * BCS + 8 * ch) = live ? breg[m] : make_uint4(0, 0, 0, 0);
            *(uint4*)(s_Ct + r * BCS + 8 * ch) = live ? cregt[m] : make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int m = 0; m < DT_PT; ++m) {
        const int e = tid + NT * m;
        const int n = e / HW, hh = e - n * HW;
        if (e < T * HW) s_dth[hh * TP + n] = (uint16_t)dtr[m];
    }
    __syncthreads();
    // C operands of the read-out MFMA
    bf16x8 creg[TI][KS];
#pragma unroll
    for (int it = 0; it < TI; ++it)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            creg[it][ks] = *(const bf16x8*)(s_Ct + (16 * it + r16) * BCS + 32 * ks + 8 * q);
    // pair scores G = C B^T on MFMA, once for all heads: the TI (TI + 1) / 2
    // lower-triangular 16 x 16 tiles (ti, tj <= ti) go round the waves in a
    // plain loop, both operands read from the LDS tiles (C rows of tile ti as
    // the A operand, B rows of tile tj as the B operand); output row 4q + r,
    // column r16 is G_ij for i = 16 ti + 4q + r, j = 16 tj + r16. Each G_ij
    // depends on C_i and B_j only.
    constexpr int kTiles = TI * (TI + 1) / 2;
    for (int tt = w; tt < kTiles; tt += 4 * HW) {
        int ti = 0, tj = tt;  // tt = ti (ti + 1) / 2 + tj
        while (tj > ti) tj -= ++ti;
        f32x4 g4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            g4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                *(const bf16x8*)(s_Ct + (16 * ti + r16) * BCS + 32 * ks + 8 * q),
                *(const bf16x8*)(s_Bt + (16 * tj + r16) * BCS + 32 * ks + 8 * q), g4, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) s_G[(16 * ti + 4 * q + r) * TP + 16 * tj + r16] = g4[r];
    }
    // this wave's x slice in its own LDS region
    uint16_t* sx = s_x[w];
#pragma unroll
    for (int m = 0; m < Cfg::kXChunks; ++m) {
        const int c = lane + kWave * m;
        const int row = c >> 1, half = c & 1;
        if (row < T) {
            uint2* dst = (uint2*)(sx + row * kXStride + 8 * half);
            dst[0] = make_uint2(xr[m].x, xr[m].y);
            dst[1] = make_uint2(xr[m].z, xr[m].w);
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- head
    // state read-out: acc[it] = (h0 C^T) tile, rows p = 16 wl + 4q + r, column
    // i; h0 is split into bf16 high and low halves, the A operand of k-step ks
    // being columns 32 ks + 8q .. + 7 of row 16 wl + r16
    bf16x8 hop[KS], lop[KS];
    if (LIN) {
        // each wave turns its runs into operands through its own 16 x N bf16
        // plane in the B/C tile memory (free since the barrier above): 16-byte
        // chunk c of row r sits at chunk c ^ (r mod chunks-per-row), so the 16
        // rows one operand read touches fall on different banks
        constexpr int CH = N / 8;  // 16-byte chunks per row of a plane
        unsigned char* plane = (unsigned char*)(s_BC + w * 16 * N);
        auto stage = [&](bool low) {
#pragma unroll
            for (int m = 0; m < 2 * KS; ++m) {
                const int e = 4 * (lane + kWave * m);  // element of the slice
                const int r = e / N, c = e % N;
                const float4 v = hr[m >> 1][m & 1];
                const float f[4] = {v.x, v.y, v.z, v.w};
                uint16_t u[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const __bf16 hb = (__bf16)f[k];
                    u[k] = __builtin_bit_cast(uint16_t, low ? (__bf16)(f[k] - (float)hb) : hb);
                }
                *(uint2*)(plane + r * 2 * N + (((c >> 3) ^ (r & (CH - 1))) << 4) + 8 * ((c >> 2) & 1)) =
                    make_uint2(u[0] | (uint32_t)u[1] << 16, u[2] | (uint32_t)u[3] << 16);
            }
            wave_sync();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 o = *(const bf16x8*)(plane + r16 * 2 * N + (((4 * ks + q) ^ (r16 & (CH - 1))) << 4));
                if (low) lop[ks] = o; else hop[ks] = o;
            }
            wave_sync();
        };
        stage(false);
        stage(true);
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) split_hi_lo(hr[ks][0], hr[ks][1], hop[ks], lop[ks]);
    }
    f32x4 acc[TI];
#pragma unroll
    for (int it = 0; it < TI; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int it = 0; it < TI; ++it) {
            acc[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hop[ks], creg[it][ks], acc[it], 0, 0, 0);
            acc[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lop[ks], creg[it][ks], acc[it], 0, 0, 0);
        }
    }

    const uint16_t* sdt = s_dth + slot * TP;
    const float Ah = A[h];
    const float Dh = D[h];
#pragma unroll
    for (int it = 0; it < TI; ++it) {
        const int i = 16 * it + r16;
        if (i >= T) continue;
        // walk up the root path of node i: the next ancestor, its step size, its
        // x row and its pair score are read in the same round
        float t0 = 0.f, t1 = 0.f, t2 = 0.f, t3 = 0.f;
        float s = 0.f;  // sum of dt*A over the path nodes from i up to (excluding) j
        const float* Gi = s_G + i * TP;
        for (int j = i; j >= 0;) {
            const int pj = s_par[j];
            const float dtj = bf16_bits_to_f32(sdt[j]);
            const float wt = Gi[j] * __expf(s) * dtj;
            const uint2 xv = *(const uint2*)(sx + j * kXStride + 4 * q);
            t0 += wt * lo_bf16(xv.x);
            t1 += wt * hi_bf16(xv.x);
            t2 += wt * lo_bf16(xv.y);
            t3 += wt * hi_bf16(xv.y);
            s += dtj * Ah;
            j = pj;
        }
        const float sc = __expf(s);
        const uint2 xi = *(const uint2*)(sx + i * kXStride + 4 * q);
        const float o0 = acc[it][0] * sc + t0 + Dh * lo_bf16(xi.x);
        const float o1 = acc[it][1] * sc + t1 + Dh * hi_bf16(xi.x);
        const float o2 = acc[it][2] * sc + t2 + Dh * lo_bf16(xi.y);
        const float o3 = acc[it][3] * sc + t3 + Dh * hi_bf16(xi.y);
        const uint2 ov = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        if (LIN) *(uint2*)(s_y + i * kYS + 16 * wl + 4 * q) = ov;
        else *(uint2*)(y + (((size_t)b * T + i) * H + h) * kP + 16 * wl + 4 * q) = ov;
    }
    if (LIN) {
        // y as whole rows: eight consecutive threads store one node's 128 bytes
        // (the per-wave 8-byte pieces cost about 2 us of the launch's memory
        // skeleton at batch 16 x 31 nodes x 80 heads)
        lds_barrier();
#pragma unroll
        for (int k = 0; k < (TP * 8 + NT - 1) / NT; ++k) {
            const int idx = tid + NT * k;
            const int row = idx >> 3, ch = idx & 7;
            if (row < T)
                *(uint4*)(y + (((size_t)b * T + row) * H + h) * kP + 8 * ch) = *(const uint4*)(s_y + row * kYS + 8 * ch);
        }
    }
}

bool verify_mfma_small_supported(int T) { return T <= 64; }

template <int TI, int KS, int HW>
static const void* small_kernel() { return (const void*)verify_mfma_kernel<TI, KS, HW>; }

template <int HW>
static const void* pick_small_hw(int T, int N) {
    const int tiles = (T + 15) / 16;
    if (N == 64)
        return tiles <= 1 ? small_kernel<1, 2, HW>() : tiles <= 2 ? small_kernel<2, 2, HW>() : small_kernel<4, 2, HW>();
    return tiles <= 1 ? small_kernel<1, 4, HW>() : tiles <= 2 ? small_kernel<2, 4, HW>() : small_kernel<4, 4, HW>();
}

hipError_t launch_verify_small(const VerifyArgs& a, int HB, hipStream_t stream) {
    // heads per work-group: the largest of 4, 2, 1 that divides the requested
    // count (results do not depend on it)
    const int hw = HB % 4 == 0 ? 4 : HB % 2 == 0 ? 2 : 1;
    const void* k = hw == 4 ? pick_small_hw<4>(a.T, a.N) : hw == 2 ? pick_small_hw<2>(a.T, a.N)
                                                                 : pick_small_hw<1>(a.T, a.N);
    dim3 grid((unsigned)(a.batch * (a.H / hw)));
    void* args[] = {(void*)&a.x, (void*)&a.dt, (void*)&a.A, (void*)&a.B, (void*)&a.C, (void*)&a.D,
                    (void*)&a.h0, (void*)&a.parent, (void*)&a.y, (void*)&a.tree_status,
                    (void*)&a.T, (void*)&a.H, (void*)&a.G};
    return hipLaunchKernel(k, grid, dim3(4 * hw * kWave), args, 0, stream);
}

}  // namespace tsv
