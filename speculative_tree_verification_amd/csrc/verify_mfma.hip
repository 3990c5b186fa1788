// verify_mfma.hip -- packed-tree verification of one Mamba2/SSD layer, bf16
// inputs, head_dim 64, d_state 64 or 128, on gfx950 matrix cores.
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
//  * work-group = (item b, block of HB heads of one group); 256 threads.
//  * set-up, once per work-group: the tree is validated and its depths found
//    by pointer jumping in LDS; the ancestor pairs (i, j) are enumerated by a
//    block scan of depth+1; G_ij is formed on those pairs only (never on the
//    dense T x T square) and kept in LDS for all HB heads.
//  * per head, wave w owns head_dim rows 16w..16w+15 and streams its own
//    16 x N slice of h0 straight from HBM into registers (each byte read once,
//    128-byte contiguous row pieces). The read-out C h0^T runs on MFMA with h0
//    split into bf16 high + low halves (about 16 significant bits); C is an
//    exact bf16 operand kept in registers (T <= 64) or LDS (T <= 256).
//  * the intra-tree term is sparse (depth+1 terms per node), so it is walked
//    along each node's root path in fp32 VALU, with exp evaluated only on
//    ancestor pairs and the decay summed along the walk (no cancellation).
//  * the next head's h0 / x / dt are loaded while the current one computes.
#include "common.hpp"
#include "launch.hpp"

namespace tsv {

constexpr int kP = 64;        // head_dim: 4 tiles of 16 rows, one per wave
constexpr int kXStride = 20;  // LDS row stride (uint16) of a wave's 16-column x slice

template <int TI>
struct MfmaCfg {
    static constexpr int TP = 16 * TI;  // node count padded to whole 16-node tiles
    static constexpr int kFullPairs = TP * (TP + 1) / 2;
    static constexpr int kMaxPairs = kFullPairs < 4096 ? kFullPairs : 4096;
    static constexpr bool kCInLds = TI > 4;
    static constexpr int kXChunks = (2 * TP + kWave - 1) / kWave;
    static constexpr int kDtChunks = (TP + kWave - 1) / kWave;
};

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// dot product of two bf16 rows of length N (multiple of 8, 16-byte aligned)
__device__ __forceinline__ float dot_bf16_row(const uint16_t* a, const uint16_t* b, int N) {
    float s = 0.f;
    for (int n = 0; n < N; n += 8) {
        uint4 va = *(const uint4*)(a + n);
        uint4 vb = *(const uint4*)(b + n);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, va.x),
                                            __builtin_bit_cast(bf16x2, vb.x), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, va.y),
                                            __builtin_bit_cast(bf16x2, vb.y), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, va.z),
                                            __builtin_bit_cast(bf16x2, vb.z), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, va.w),
                                            __builtin_bit_cast(bf16x2, vb.w), s, false);
    }
    return s;
}

template <int TI, int KS>
__global__ __launch_bounds__(kBlock) void verify_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const float* __restrict__ D, const float* __restrict__ h0, const int32_t* __restrict__ parent,
    uint16_t* __restrict__ y, int32_t* __restrict__ tree_status, int T, int H, int G, int HB) {
    using Cfg = MfmaCfg<TI>;
    constexpr int N = 32 * KS;
    constexpr int TP = Cfg::TP;
    constexpr int MAXP = Cfg::kMaxPairs;
    constexpr int CST = N + 8;  // LDS row stride of C (bf16): 16-byte pad against bank conflicts

    __shared__ int s_par[kMaxNodes];
    __shared__ int s_nxt[kMaxNodes];
    __shared__ int s_dep[kMaxNodes];
    __shared__ int s_off[kMaxNodes];
    __shared__ int s_scan[4];
    __shared__ uint16_t s_pair[MAXP];  // node i in the low byte, ancestor j in the high byte
    __shared__ float s_G[MAXP];
    __shared__ __attribute__((aligned(16))) uint16_t s_x[4][TP * kXStride];
    __shared__ float s_dtw[4][TP];
    __shared__ __attribute__((aligned(16))) uint16_t s_C[Cfg::kCInLds ? TP * CST : 8];

    const int nblk = H / HB;
    const int b = blockIdx.x / nblk;
    const int h_first = (blockIdx.x % nblk) * HB;
    const int g = h_first / (H / G);
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int r16 = lane & 15;
    const int q = lane >> 4;

    // ---------------------------------------------------------------- set-up
    const int st = load_tree(parent + (size_t)b * T, T, s_par);
    if (h_first == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st) return;

    const int dep = tree_depth(s_par, T, s_nxt, s_dep);
    int total_pairs;
    const int off = block_exclusive_scan(tid < T ? dep + 1 : 0, s_scan, &total_pairs);
    const bool cached = total_pairs <= MAXP;
    if (tid < T) {
        s_off[tid] = off;
        if (cached) {
            int k = 0;
            for (int j = tid; j >= 0; j = s_par[j]) s_pair[off + k++] = (uint16_t)(tid | (j << 8));
        }
    }
    const size_t bc_row0 = ((size_t)b * T) * G + g;  // row (b, node 0, g) of B and C
    if constexpr (Cfg::kCInLds) {
        constexpr int kChunksPerRow = N / 8;
        for (int c = tid; c < TP * kChunksPerRow; c += kBlock) {
            const int row = c / kChunksPerRow, col = (c % kChunksPerRow) * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row < T) v = *(const uint4*)(Cm + (bc_row0 + (size_t)row * G) * N + col);
            *(uint4*)(s_C + row * CST + col) = v;
        }
    }
    __syncthreads();
    if (cached) {
        for (int pq = tid; pq < total_pairs; pq += kBlock) {
            const int pr = s_pair[pq];
            const int i = pr & 255, j = pr >> 8;
            const uint16_t* Ci;
            if constexpr (Cfg::kCInLds)
                Ci = s_C + i * CST;
            else
                Ci = Cm + (bc_row0 + (size_t)i * G) * N;
            s_G[pq] = dot_bf16_row(Ci, Bm + (bc_row0 + (size_t)j * G) * N, N);
        }
    }
    bf16x8 creg[Cfg::kCInLds ? 1 : TI][KS];
    if constexpr (!Cfg::kCInLds) {
#pragma unroll
        for (int it = 0; it < TI; ++it) {
            const int i = 16 * it + r16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint4 v = make_uint4(0, 0, 0, 0);
                if (i < T) v = *(const uint4*)(Cm + (bc_row0 + (size_t)i * G) * N + 32 * ks + 8 * q);
                creg[it][ks] = __builtin_bit_cast(bf16x8, v);
            }
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- heads
    uint16_t* sx = s_x[w];
    float* sdt = s_dtw[w];
    float4 hr[KS][2];
    uint4 xr[Cfg::kXChunks];
    uint32_t dr[Cfg::kDtChunks];

    auto load_head = [&](int h) {
        const float* hrow = h0 + (((size_t)b * H + h) * kP + 16 * w + r16) * N + 8 * q;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            hr[ks][0] = *(const float4*)(hrow + 32 * ks);
            hr[ks][1] = *(const float4*)(hrow + 32 * ks + 4);
        }
#pragma unroll
        for (int m = 0; m < Cfg::kXChunks; ++m) {
            const int c = lane + kWave * m;
            const int row = c >> 1, half = c & 1;
            xr[m] = make_uint4(0, 0, 0, 0);
            if (row < T)
                xr[m] = *(const uint4*)(x + (((size_t)b * T + row) * H + h) * kP + 16 * w + 8 * half);
        }
#pragma unroll
        for (int m = 0; m < Cfg::kDtChunks; ++m) {
            const int i = lane + kWave * m;
            dr[m] = (i < T) ? dt[((size_t)b * T + i) * H + h] : 0u;
        }
    };

    load_head(h_first);
    for (int hh = 0; hh < HB; ++hh) {
        const int h = h_first + hh;
        // stage this head's x slice and dt in the wave's own LDS region
        wave_sync();
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
#pragma unroll
        for (int m = 0; m < Cfg::kDtChunks; ++m) {
            const int i = lane + kWave * m;
            if (i < T) sdt[i] = bf16_bits_to_f32(dr[m]);
        }
        // h0 rows -> bf16 high and low parts (h0 ~= hi + lo to ~2^-16 relative)
        bf16x8 hi[KS], lo[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float f[8] = {hr[ks][0].x, hr[ks][0].y, hr[ks][0].z, hr[ks][0].w,
                                hr[ks][1].x, hr[ks][1].y, hr[ks][1].z, hr[ks][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 hb = (__bf16)f[e];
                hi[ks][e] = hb;
                lo[ks][e] = (__bf16)(f[e] - (float)hb);
            }
        }
        if (hh + 1 < HB) load_head(h + 1);
        wave_sync();

        // state read-out: acc[it] = (h0 C^T) tile, rows p = 16w + 4q + r, column i
        f32x4 acc[TI];
#pragma unroll
        for (int it = 0; it < TI; ++it) {
            acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 bop;
                if constexpr (Cfg::kCInLds)
                    bop = *(const bf16x8*)(s_C + (16 * it + r16) * CST + 32 * ks + 8 * q);
                else
                    bop = creg[it][ks];
                acc[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[ks], bop, acc[it], 0, 0, 0);
                acc[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[ks], bop, acc[it], 0, 0, 0);
            }
        }

        const float Ah = A[h];
        const float Dh = D[h];
#pragma unroll
        for (int it = 0; it < TI; ++it) {
            const int i = 16 * it + r16;
            if (i >= T) continue;
            float t0 = 0.f, t1 = 0.f, t2 = 0.f, t3 = 0.f;
            float s = 0.f;  // sum of dt*A over the nodes from i up to (excluding) j
            int k = 0;
            const int base = s_off[i];
            for (int j = i; j >= 0; j = s_par[j], ++k) {
                const float dtj = sdt[j];
                float gij;
                if (cached)
                    gij = s_G[base + k];
                else
                    gij = dot_bf16_row(Cm + (bc_row0 + (size_t)i * G) * N,
                                       Bm + (bc_row0 + (size_t)j * G) * N, N);
                const float wt = gij * __expf(s) * dtj;
                const uint2 xv = *(const uint2*)(sx + j * kXStride + 4 * q);
                t0 += wt * lo_bf16(xv.x);
                t1 += wt * hi_bf16(xv.x);
                t2 += wt * lo_bf16(xv.y);
                t3 += wt * hi_bf16(xv.y);
                s += dtj * Ah;
            }
            const float sc = __expf(s);
            const uint2 xi = *(const uint2*)(sx + i * kXStride + 4 * q);
            const float o0 = acc[it][0] * sc + t0 + Dh * lo_bf16(xi.x);
            const float o1 = acc[it][1] * sc + t1 + Dh * hi_bf16(xi.x);
            const float o2 = acc[it][2] * sc + t2 + Dh * lo_bf16(xi.y);
            const float o3 = acc[it][3] * sc + t3 + Dh * hi_bf16(xi.y);
            *(uint2*)(y + (((size_t)b * T + i) * H + h) * kP + 16 * w + 4 * q) =
                make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        }
    }
}

bool verify_mfma_supported(int P, int N) { return P == kP && (N == 64 || N == 128); }

int verify_mfma_default_heads_per_block(int batch, int T, int H, int G) {
    // largest divisor of the heads per group that still gives >= 4 work-groups per CU
    const int hpg = H / G;
    int best = 1;
    for (int d = 1; d <= hpg; ++d)
        if (hpg % d == 0 && (long)batch * (H / d) >= 1024) best = d;
    (void)T;
    return best;
}

template <int TI, int KS>
static void launch_one(const VerifyArgs& a, int HB, hipStream_t stream) {
    dim3 grid((unsigned)(a.batch * (a.H / HB)));
    hipLaunchKernelGGL((verify_mfma_kernel<TI, KS>), grid, dim3(kBlock), 0, stream,
                       (const uint16_t*)a.x, (const uint16_t*)a.dt, a.A, (const uint16_t*)a.B,
                       (const uint16_t*)a.C, a.D, a.h0, a.parent, (uint16_t*)a.y, a.tree_status,
                       a.T, a.H, a.G, HB);
}

template <int KS>
static void launch_ks(const VerifyArgs& a, int HB, hipStream_t stream) {
    const int tiles = (a.T + 15) / 16;
    if (tiles <= 1)
        launch_one<1, KS>(a, HB, stream);
    else if (tiles <= 2)
        launch_one<2, KS>(a, HB, stream);
    else if (tiles <= 4)
        launch_one<4, KS>(a, HB, stream);
    else if (tiles <= 8)
        launch_one<8, KS>(a, HB, stream);
    else
        launch_one<16, KS>(a, HB, stream);
}

hipError_t launch_verify_mfma(const VerifyArgs& a, int heads_per_block, hipStream_t stream) {
    const int HB = heads_per_block > 0 ? heads_per_block
                                       : verify_mfma_default_heads_per_block(a.batch, a.T, a.H, a.G);
    if (a.N == 64)
        launch_ks<2>(a, HB, stream);
    else
        launch_ks<4>(a, HB, stream);
    return hipGetLastError();
}

}  // namespace tsv
