// large.hip -- verify of one SSD layer over packed trees of 257 to 1024 nodes
// ("STree: Speculative Tree Decoding for Hybrid State Space Models",
// atlas.scime.ai summary, section "Approach": the accumulated log transitions
// along ancestor paths give every node its own path's output in one pass).
// The commit of such trees is the commit kernel of commit.hip with four nodes
// per thread.
//
// Same outputs as the kernels for trees of up to 256 nodes. The plain kernel
// below takes fp32 VALU arithmetic, any head_dim and d_state up to 256, both
// input dtypes; the MFMA kernel further down takes bf16 Mamba2 head shapes.
//
// Verify: one work-group of 1024 threads (16 waves) per (item, head), one
// thread per node for the tree check. Each wave takes every 16th node; its 64
// lanes hold the node's C row spread over d_state, so each ancestor's score
// C_i . B_j is one reduction across the wave, and the node's outputs spread
// over head_dim (lane p and p + 64k). The decay from ancestor j to i is summed
// along the walk (no difference of prefix sums); the walk requests the rows of
// kWalk ancestors at a time. The h0 read-out takes h0 from LDS (rows padded
// by 4 floats, read 4 columns at a time against the node's C row, which the
// wave keeps in LDS too) when a head's block fits in 64 KiB.
#include "common.hpp"
#include "launch.hpp"

namespace tsv {

constexpr int kLargeThreads = kMaxNodesLarge;  // one thread per node for the tree check
constexpr int kLargeWaves = kLargeThreads / kWave;
constexpr int kLargeH0Lds = 16384;  // floats of h0 staged in LDS (64 KiB)
constexpr int kWalk = 8;            // ancestors whose rows are requested together
constexpr int kMaxDimLarge = 256;

// NK, PK: registers per lane for d_state (lane + 64 k, k < NK) and head_dim
template <typename TIO, bool H0LDS, int NK, int PK>
__global__ __launch_bounds__(kLargeThreads) void verify_large_kernel(
    const TIO* __restrict__ x, const TIO* __restrict__ dt, const float* __restrict__ A,
    const TIO* __restrict__ Bm, const TIO* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ h0, const int32_t* __restrict__ parent, TIO* __restrict__ y,
    int32_t* __restrict__ tree_status, int T, int H, int P, int N, int G) {
    __shared__ int s_par[kMaxNodesLarge];
    __shared__ float s_dt[kMaxNodesLarge];
    __shared__ __attribute__((aligned(16))) float s_h0[H0LDS ? kLargeH0Lds : 1];  // [p][N + 4]
    __shared__ __attribute__((aligned(16))) float s_c[kLargeWaves][kMaxDimLarge];  // each wave's C row

    const int b = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int st = load_tree(parent + (size_t)b * T, T, s_par);
    if (h == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st) return;

    const float Ah = A[h];
    const float Dh = D[h];
    const float* H0 = h0 + ((size_t)b * H + h) * P * N;
    for (int i = tid; i < T; i += kLargeThreads) s_dt[i] = Elem<TIO>::ld(dt, ((size_t)b * T + i) * H + h);
    const int NS = ((N + 3) & ~3) + 4;  // padded h0 row, a multiple of 4 floats
    if (H0LDS)
        for (int e = tid; e < P * N; e += kLargeThreads) {
            const int p = e / N, n = e - p * N;
            s_h0[p * NS + n] = H0[e];
        }
    __syncthreads();

    const size_t xrow = (size_t)H * P;  // x / y stride between nodes
    const TIO* xb = x + ((size_t)b * T * H + h) * P;
    for (int i = w; i < T; i += kLargeWaves) {
        const TIO* Ci = Cm + (((size_t)b * T + i) * G + g) * N;
        float c[NK];  // C_i[lane + 64 k]
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            c[k] = lane + 64 * k < N ? Elem<TIO>::ld(Ci, lane + 64 * k) : 0.f;
            s_c[w][lane + 64 * k] = c[k];
        }
        float acc[PK];  // output p = lane + 64 k
#pragma unroll
        for (int k = 0; k < PK; ++k) acc[k] = 0.f;
        float s = 0.f;  // sum of dt A over the nodes from i up to (excluding) j
        // the walk, kWalk ancestors at a time: their indices from the parents in
        // LDS, then every B and x load of the batch before the first use, so a
        // batch costs one memory round trip
        for (int j = i; j >= 0;) {
            int js[kWalk];
#pragma unroll
            for (int u = 0; u < kWalk; ++u) {
                js[u] = j;
                j = j >= 0 ? s_par[j] : -1;
            }
            float bv[kWalk][NK], xv[kWalk][PK];
#pragma unroll
            for (int u = 0; u < kWalk; ++u) {
                const int ju = max(js[u], 0);
                const TIO* Bj = Bm + (((size_t)b * T + ju) * G + g) * N;
#pragma unroll
                for (int k = 0; k < NK; ++k)
                    bv[u][k] = lane + 64 * k < N ? Elem<TIO>::ld(Bj, lane + 64 * k) : 0.f;
#pragma unroll
                for (int k = 0; k < PK; ++k)
                    xv[u][k] = lane + 64 * k < P ? Elem<TIO>::ld(xb, ju * xrow + lane + 64 * k) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kWalk; ++u) {
                if (js[u] < 0) break;  // wave-uniform
                float gp = 0.f;
#pragma unroll
                for (int k = 0; k < NK; ++k) gp += c[k] * bv[u][k];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) gp += __shfl_xor(gp, off, kWave);
                const float dtj = s_dt[js[u]];
                const float wgt = gp * expf(s) * dtj;
#pragma unroll
                for (int k = 0; k < PK; ++k) acc[k] += wgt * xv[u][k];
                s += dtj * Ah;
            }
        }
        const float ei = expf(s);
        wave_sync();  // the wave's C row in LDS
        // read-out h0 . C_i, four columns at a time
        const int N4 = N & ~3;
#pragma unroll
        for (int k = 0; k < PK; ++k) {
            if (64 * k >= P) break;  // wave-uniform
            const int p = min(lane + 64 * k, P - 1);
            float ch = 0.f;
            if (H0LDS) {
                const float* hr = s_h0 + p * NS;
#pragma unroll 8
                for (int n = 0; n < N4; n += 4) {
                    const float4 cv = *(const float4*)&s_c[w][n];
                    const float4 hv = *(const float4*)&hr[n];
                    ch += cv.x * hv.x + cv.y * hv.y + cv.z * hv.z + cv.w * hv.w;
                }
                for (int n = N4; n < N; ++n) ch += s_c[w][n] * hr[n];
            } else {
                const float* hr = H0 + (size_t)p * N;
                for (int n = 0; n < N; ++n) ch += s_c[w][n] * hr[n];
            }
            if (lane + 64 * k < P) {
                const size_t o = i * xrow + lane + 64 * k;
                Elem<TIO>::st(y + ((size_t)b * T * H + h) * P, o, ei * ch + acc[k] + Dh * Elem<TIO>::ld(xb, o));
            }
        }
        wave_sync();  // C row consumed before the next node writes it
    }
}

// ----------------------------------------------------------------------------
// MFMA form for bf16 inputs, head_dim 64, d_state 32 KS (64 or 128). Each wave
// takes tiles of 16 consecutive nodes:
//  - read-out h0 . C_i of the tile on bf16 MFMA (h0 as bf16 high and low
//    parts in LDS, C rows as the A operand);
//  - the ancestors of the tile's nodes, 32 steps of each root path at a time:
//    node lanes walk the parents in LDS, record each ancestor by distance with
//    its decay exp(sum of dt A from i up to, not including, j) dt_j, and flag
//    it; the flags are compacted into the column list J (no repeats);
//  - per block of 16 columns: G^T = B[J] C[tile]^T on bf16 MFMA, masked to the
//    recorded (node, ancestor) pairs and weighted by their decays (S), then
//    S X[J] on fp32 MFMA. The accumulator of G^T holds S[i][j] with i = lane % 16
//    and j = 4 (lane / 16) + c in element c: the A operand of the step that
//    takes those j, with the matching X rows as its B operand.
constexpr int kLmDist = 32;  // path steps per pass

template <int KS>
__global__ __launch_bounds__(kLargeThreads) void verify_large_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ h0, const int32_t* __restrict__ parent, uint16_t* __restrict__ y,
    int32_t* __restrict__ tree_status, int T, int H, int G, int S) {
    constexpr int P = 64, N = 32 * KS, NW = kLargeWaves;
    constexpr int RH = N + 8;  // row stride (bf16) of the h0 planes
    __shared__ int s_par[kMaxNodesLarge];
    __shared__ int s_dep[kMaxNodesLarge];
    __shared__ int s_nxt[kMaxNodesLarge];
    __shared__ int s_red[kLargeWaves];
    __shared__ float s_a[kMaxNodesLarge];  // dt of each node
    __shared__ __attribute__((aligned(16))) uint16_t s_h0h[P * RH];
    __shared__ __attribute__((aligned(16))) uint16_t s_h0l[P * RH];
    // distance-major, so that the 16 node lanes of a walk step write 16
    // neighbouring entries (rows per node put 4 or 8 of them on one LDS bank)
    __shared__ uint16_t s_path[NW][kLmDist][16];  // ancestor at distance 32 k + t of tile node r
    __shared__ float s_dec[NW][kLmDist][16];      // its decay times its dt
    __shared__ float s_cum[NW][16];               // cum of tile node r
    __shared__ int s_plen[NW][16];                // entries of this pass for tile node r
    __shared__ unsigned long long s_bits[NW][kMaxNodesLarge / 64];  // ancestors flagged this pass
    __shared__ uint16_t s_J[NW][16 * kLmDist];

    // logical block = (b H + h) S + part: the S work-groups of one (item, head)
    // take every S-th node tile (shallow and deep ones alike) and share an XCD,
    // so that h0 is fetched into one L2
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int part = lb % S;
    const int b = lb / S / H;
    const int h = lb / S % H;
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane & 15, q4 = lane >> 4;
    // the parents, this thread's step size and its share of h0 leave together
    // (one thread per node, T <= 1024 = threads); the tree check and the depths
    // use LDS-only barriers, so they overlap the other two round trips
    const int par_i = load_parent(parent + (size_t)b * T, T);
    const uint32_t dt_i = gload(dt + ((size_t)b * T + min(tid, T - 1)) * H + h);
    constexpr int HF4 = P * N / 4 / kLargeThreads;  // float4 of h0 per thread
    static_assert(P * N % (4 * kLargeThreads) == 0, "h0 must split evenly over the threads");
    float4 hv[HF4];
    const float4* H0 = (const float4*)(h0 + ((size_t)b * H + h) * P * N);
#pragma unroll
    for (int m = 0; m < HF4; ++m) hv[m] = gload(H0 + tid + kLargeThreads * m);
    const int st = check_tree_lds<kLargeThreads>(par_i, T, s_par, s_red);
    if (h == 0 && part == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st) return;
    // depths: a walk to the root per node, pointer jumping past 16 levels
    const int dep_i = tree_depth_shallow<kLargeThreads>(s_par, T, s_nxt, s_dep, s_red);
    if (tid < T) s_dep[tid] = dep_i;

    const float Ah = A[h];
    const float Dh = D[h];
    if (tid < T) s_a[tid] = bf16_bits_to_f32(dt_i);
#pragma unroll
    for (int m = 0; m < HF4; ++m) {
        const int e = 4 * (tid + kLargeThreads * m);  // 4 consecutive n of row p
        const int p = e / N, n = e - p * N;
        const float v[4] = {hv[m].x, hv[m].y, hv[m].z, hv[m].w};
        uint16_t hb[4], lb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const __bf16 t = (__bf16)v[k];
            hb[k] = __builtin_bit_cast(uint16_t, t);
            lb[k] = f32_to_bf16_bits(v[k] - (float)t);
        }
        *(uint2*)&s_h0h[p * RH + n] = make_uint2(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16));
        *(uint2*)&s_h0l[p * RH + n] = make_uint2(lb[0] | ((uint32_t)lb[1] << 16), lb[2] | ((uint32_t)lb[3] << 16));
    }
    for (int e = tid; e < NW * kMaxNodesLarge / 64; e += kLargeThreads) (&s_bits[0][0])[e] = 0ull;
    __syncthreads();

    // rows within an item are addressed by 32-bit offsets from the item's base
    const uint32_t xrow = (uint32_t)(H * P);  // x / y stride between nodes
    const uint32_t bcrow = (uint32_t)(G * N);
    const uint16_t* xb = x + ((size_t)b * T * H + h) * P;
    uint16_t* yb = y + ((size_t)b * T * H + h) * P;
    const uint16_t* Bb = Bm + ((size_t)b * T * G + g) * N;
    const uint16_t* Cb = Cm + ((size_t)b * T * G + g) * N;
    for (int tt = w; 16 * (tt * S + part) < T; tt += NW) {
        const int i0 = 16 * (tt * S + part);
        // C rows of the tile: node i0 + l16, columns 32 ks + 8 q4 ..
        bf16x8 cf[KS];
        const uint16_t* crow = Cb + (uint32_t)min(i0 + l16, T - 1) * bcrow;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) cf[ks] = __builtin_bit_cast(bf16x8, *(const uint4*)(crow + 32 * ks + 8 * q4));
        f32x4 yw[4];  // walk term: rows i0 + 4 q4 + c, columns p = 16 pt + l16
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) yw[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // the walk, 32 path steps a pass
        int jw = lane < 16 && i0 + lane < T ? i0 + lane : -1;
        float sw = 0.f;
        const int inode = i0 + l16;
        const int di = s_dep[min(inode, T - 1)];
        for (int k = 0;; ++k) {
            if (lane < 16) {
                int t = 0;
                for (; t < kLmDist && jw >= 0; ++t) {
                    const float dtj = s_a[jw];
                    s_path[w][t][lane] = (uint16_t)jw;
                    s_dec[w][t][lane] = __expf(sw) * dtj;
                    sw += dtj * Ah;
                    // flag jw unless the lane to the left (same step) has it
                    // already: neighbouring nodes share most ancestors, and
                    // atomics on one word from many lanes are serialised
                    const int left = __builtin_amdgcn_update_dpp(-2, jw, 0x111, 0xf, 0xf, false);  // row_shr:1
                    if (jw != left) atomicOr(&s_bits[w][jw >> 6], 1ull << (jw & 63));
                    jw = s_par[jw];
                }
                s_plen[w][lane] = t;
                s_cum[w][lane] = sw;
            }
            wave_sync();
            // compact the flagged ancestors (they precede the tile's last node):
            // lane wd reads word wd (one LDS round trip for all) and clears it
            // for the next pass; the non-empty words are then taken in order
            int nJ = 0;  // wave-uniform
            const int nwords = (min(T, i0 + 16) + 63) >> 6;  // at most 16
            unsigned long long myw = 0ull;
            if (lane < nwords) {
                myw = s_bits[w][lane];
                s_bits[w][lane] = 0ull;
            }
            for (unsigned long long nz = __ballot(myw != 0ull); nz; nz &= nz - 1) {
                const int wd = __builtin_ctzll(nz);  // wave-uniform
                const unsigned long long m =
                    (unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)myw, wd) |
                    ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(myw >> 32), wd) << 32);
                if ((m >> lane) & 1ull) s_J[w][nJ + __popcll(m & ((1ull << lane) - 1))] = (uint16_t)(64 * wd + lane);
                nJ += __popcll(m);
            }
            wave_sync();
            // per column block of 16: the X values this lane feeds to the S X
            // steps (row J[c0 + 4 q4 + c], column 16 pt + l16), requested with
            // the block's B rows (clamped rows past the list: loaded, unused).
            // Requesting them a block ahead needs a copy at the end of each
            // block, which waits for them there: 90.3 against 87.9 us on the
            // 1023-node trees.
            auto xvals = [&](int c0, float (&xq)[4][4]) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint16_t* xr = xb + (uint32_t)s_J[w][min(c0 + 4 * q4 + c, nJ - 1)] * xrow;
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) xq[c][pt] = bf16_bits_to_f32(xr[16 * pt + l16]);
                }
            };
            const int plen = s_plen[w][l16];  // entries of this pass for node l16
            for (int c0 = 0; c0 < nJ; c0 += 16) {
                // G^T block: rows J[c0 + l16] (A operand: B rows), columns the tile (C rows)
                const uint16_t* brow = Bb + (uint32_t)s_J[w][min(c0 + l16, nJ - 1)] * bcrow;
                uint4 bq[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) bq[ks] = *(const uint4*)(brow + 32 * ks + 8 * q4);
                float xq[4][4];
                xvals(c0, xq);
                // this lane's four columns j are kept where j is node l16's
                // ancestor at distance t of this pass, weighted by its decay;
                // each stage's LDS reads leave for all four columns together
                // (from clamped positions) and the test is a select
                int jt[4];  // j | clamped t << 16, bit 31 where t is an entry of this pass
#pragma unroll
                for (int c = 0; c < 4; ++c) jt[c] = s_J[w][min(c0 + 4 * q4 + c, nJ - 1)];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int t = di - s_dep[jt[c]] - kLmDist * k;
                    const bool ok = c0 + 4 * q4 + c < nJ && inode < T && t >= 0 && t < plen;
                    jt[c] |= (min(max(t, 0), kLmDist - 1) << 16) | (ok ? (int)0x80000000 : 0);
                }
                int pj[4];
                float dj[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int t = (jt[c] >> 16) & (kLmDist - 1);
                    pj[c] = s_path[w][t][l16];
                    dj[c] = s_dec[w][t][l16];
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(pj[c]), "+v"(dj[c]));  // all reads before the tests
                f32x4 gt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    gt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bq[ks]), cf[ks], gt, 0, 0, 0);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float wgt = (jt[c] < 0 && pj[c] == (jt[c] & 0xffff)) ? dj[c] : 0.f;
                    const float sv = gt[c] * wgt;
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt)
                        yw[pt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sv, xq[c][pt], yw[pt], 0, 0, 0);
                }
            }
            if (!__ballot(lane < 16 && jw >= 0)) break;
            wave_sync();  // lists and columns of this pass consumed
        }
        // own x values for the D term, requested before the read-out
        float xi[4][4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int i = min(i0 + 4 * q4 + c, T - 1);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) xi[c][pt] = bf16_bits_to_f32(xb[(uint32_t)i * xrow + 16 * pt + l16]);
        }
        // read-out h0 . C of the tile, same layout as the walk term
        f32x4 y0[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            y0[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int o = (16 * pt + l16) * RH + 32 * ks + 8 * q4;
                y0[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cf[ks], *(const bf16x8*)&s_h0l[o], y0[pt], 0, 0, 0);
                y0[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cf[ks], *(const bf16x8*)&s_h0h[o], y0[pt], 0, 0, 0);
            }
        }
        wave_sync();  // s_cum
        // y of the tile leaves through this wave's decay table (free once the
        // walk is done; 16 rows x 128 bytes, row-major, so every write below
        // is the lane's base plus a constant) as two 16-byte stores per lane
        // instead of sixteen 2-byte ones
        uint16_t* ty = (uint16_t*)&s_dec[w][0][0];
        uint16_t* tyl = ty + 4 * q4 * P + l16;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (i0 + 4 * q4 + c < T) {
                const float ec = __expf(s_cum[w][4 * q4 + c]);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    tyl[c * P + 16 * pt] = f32_to_bf16_bits(ec * y0[pt][c] + yw[pt][c] + Dh * xi[c][pt]);
            }
        }
        wave_sync();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int k = lane + kWave * k2;
            const int r = k >> 3, ch = k & 7;
            if (i0 + r < T) *(uint4*)(yb + (uint32_t)(i0 + r) * xrow + 8 * ch) = *(const uint4*)(ty + 8 * k);
        }
        wave_sync();  // s_cum, lists and the y tile of this tile consumed
    }
}

// Work-groups per (item, head) of the MFMA kernel: a work-group fills a
// compute unit, so the launch runs in rounds of one work-group per unit. Each
// of the S parts takes every S-th 16-node tile (at least one per wave) and
// repeats the set-up (tree, depth, h0 planes), which costs about a fifth of
// an unsplit work-group's tile work on the 1023-node trees. S minimises
// rounds x (set-up + tile work / S) = ceil(units S / CUs) (0.2 + 1 / S).
constexpr double kLargeSetupShare = 0.2;
static int large_split(int units, int T) {
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int tiles = (T + 15) / 16;
    int best = 1;
    double best_cost = 1e30;
    for (int S = 1; S <= 8 && S * kLargeWaves <= tiles; S *= 2) {
        const double cost = (double)(((long)units * S + cus - 1) / cus) * (kLargeSetupShare + 1.0 / S);
        if (cost < best_cost) best_cost = cost, best = S;
    }
    return best;
}

hipError_t launch_verify_large(const VerifyArgs& a, bool bf16, hipStream_t stream) {
    dim3 grid((unsigned)(a.batch * a.H));
    if (bf16 && a.P == 64 && (a.N == 64 || a.N == 128)) {
        const int S = large_split(a.batch * a.H, a.T);
        dim3 gs((unsigned)(a.batch * a.H * S));
        if (a.N == 128)
            hipLaunchKernelGGL(verify_large_mfma_kernel<4>, gs, dim3(kLargeThreads), 0, stream,
                               (const uint16_t*)a.x, (const uint16_t*)a.dt, a.A, (const uint16_t*)a.B,
                               (const uint16_t*)a.C, a.D, a.h0, a.parent, (uint16_t*)a.y,
                               a.tree_status, a.T, a.H, a.G, S);
        else
            hipLaunchKernelGGL(verify_large_mfma_kernel<2>, gs, dim3(kLargeThreads), 0, stream,
                               (const uint16_t*)a.x, (const uint16_t*)a.dt, a.A, (const uint16_t*)a.B,
                               (const uint16_t*)a.C, a.D, a.h0, a.parent, (uint16_t*)a.y,
                               a.tree_status, a.T, a.H, a.G, S);
        return hipGetLastError();
    }
    const bool lds = a.P * (((a.N + 3) & ~3) + 4) <= kLargeH0Lds;
    const bool small = a.N <= 128 && a.P <= 64;
#define TSV_LARGE(TIO, L, NK, PK)                                                                  \
    hipLaunchKernelGGL((verify_large_kernel<TIO, L, NK, PK>), grid, dim3(kLargeThreads), 0, stream, \
                       (const TIO*)a.x, (const TIO*)a.dt, a.A, (const TIO*)a.B, (const TIO*)a.C,   \
                       a.D, a.h0, a.parent, (TIO*)a.y, a.tree_status, a.T, a.H, a.P, a.N, a.G)
    if (bf16) {
        if (small) TSV_LARGE(uint16_t, true, 2, 1);
        else if (lds) TSV_LARGE(uint16_t, true, 4, 4);
        else TSV_LARGE(uint16_t, false, 4, 4);
    } else {
        if (small) TSV_LARGE(float, true, 2, 1);
        else if (lds) TSV_LARGE(float, true, 4, 4);
        else TSV_LARGE(float, false, 4, 4);
    }
#undef TSV_LARGE
    return hipGetLastError();
}

}  // namespace tsv
