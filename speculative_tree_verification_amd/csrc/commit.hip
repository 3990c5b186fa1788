// commit.hip -- rebuild, in place, the state at the end of the accepted root
// path by replaying the accepted tokens ("STree: Speculative Tree Decoding for
// Hybrid State Space Models", atlas.scime.ai summary, section "Approach": the
// state is restored from the retained activations, not from stored per-node
// states). For the path j_0 = 0, ..., j_{L-1} = l:
//   H' = exp(c_0) h0 + sum_k exp(c_{k+1}) dt_{j_k} x_{j_k} (outer) B_{j_k},
// with c_k = sum_{m >= k} dt_{j_m} A the log decay from token j_k to the end
// of the path (suffix sums, so no cancellation).
//
// Work-group = (layer, batch item, head, chunk of the P x N state); the layer
// is 0 for a single-layer call, and for a multi-layer call the work-group reads
// its layer's operand pointers from the caller's table. The path indices and
// the parents leave first (the accepted row without waiting for its length),
// then the state chunk; the tree and the path are validated bit-exactly from
// LDS behind LDS-only barriers, so dt, x and B of the path rows are requested
// while the state chunk is still in flight (their round trip overlaps the
// state's). The state is streamed once: each element is read and written by
// the same thread (rank-L update in registers), with nontemporal loads and
// stores, so that it does not displace the rows and indices that every
// work-group of a layer re-reads (the 64-layer commit of the 15-node tree
// went from 62.9 to 56.6 us with them, batch 16 x 31 nodes from 22.4 to 17.9,
// batch 32 x 63 nodes from 20.8 to 16.8, batch 64 x 255 nodes from 66.3 to
// 60.0, each measured in one process against the same build without). Invalid items leave h0
// untouched. For small trees (one 16-byte piece of x and B rows per thread
// covers every node) the rows of all nodes are requested in the first round
// trip instead, and the path's rows are picked from registers after
// validation: no second round trip (the 64-layer commit of the 15-node tree:
// 69.4 -> 62.9 us). The x rows of the other nodes cost a few percent of the
// state's traffic there (T <= N / 4); two pieces per thread (the 31- and
// 63-node trees) needed 118 registers and ran no faster.
#include "common.hpp"
#include "launch.hpp"

namespace tsv {

constexpr int kPathChunk = 16;  // path entries staged in LDS at a time
constexpr int kVec = 4;         // float4 per thread per work-group

// eight bf16 values (one 16-byte piece of a row) to fp32 in LDS
__device__ __forceinline__ void put8(float* dst, uint4 v) {
    *(float4*)dst = make_float4(bf16_bits_to_f32(v.x & 0xffff), bf16_bits_to_f32(v.x >> 16),
                                bf16_bits_to_f32(v.y & 0xffff), bf16_bits_to_f32(v.y >> 16));
    *(float4*)(dst + 4) = make_float4(bf16_bits_to_f32(v.z & 0xffff), bf16_bits_to_f32(v.z >> 16),
                                      bf16_bits_to_f32(v.w & 0xffff), bf16_bits_to_f32(v.w >> 16));
}

// NPT: tree nodes (and path entries) per thread, 1 for trees of up to 256
// nodes, 4 for up to 1024
template <typename TIO, bool VEC, bool PRE, int NPT>
__global__ __launch_bounds__(kBlock) void commit_kernel(
    const TIO* __restrict__ x_arg, const TIO* __restrict__ dt_arg, const float* __restrict__ A_arg,
    const TIO* __restrict__ B_arg, float* __restrict__ h_arg, const tsv_commit_layer* __restrict__ layers,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ accepted_len, int32_t* __restrict__ tree_status, int BH, int T,
    int H, int P, int N, int G, int Lmax, int chunks) {
    constexpr int NMAX = kBlock * NPT;
    static_assert(!PRE || NPT == 1, "preloaded rows need one node per thread");
    __shared__ int s_par[NMAX];
    __shared__ int s_path[NMAX];
    __shared__ int s_pos[PRE ? kMaxNodes : 1];  // path position of each node, or -1 (PRE)
    __shared__ float s_w[NMAX];
    __shared__ float s_w0;
    __shared__ int s_red[kBlock / kWave];
    // [kPathChunk][P] x rows, then [kPathChunk][N] B rows, of the path
    extern __shared__ __attribute__((aligned(16))) float s_dyn[];
    float* s_wx = s_dyn;
    float* s_B = s_dyn + kPathChunk * P;

    const int chunk = blockIdx.x % chunks;
    const int bh = (blockIdx.x / chunks) % BH;
    const int layer = blockIdx.x / (chunks * BH);
    const TIO* __restrict__ x = x_arg;
    const TIO* __restrict__ dt = dt_arg;
    const float* __restrict__ A = A_arg;
    const TIO* __restrict__ Bm = B_arg;
    float* __restrict__ h = h_arg;
    if (layers) {  // uniform over the launch
        const tsv_commit_layer L = layers[layer];
        x = (const TIO*)L.x;
        dt = (const TIO*)L.dt;
        A = L.A;
        Bm = (const TIO*)L.B;
        h = L.h0_inout;
    }
    const int b = bh / H;
    const int hd = bh % H;
    const int g = hd / (H / G);
    const int tid = threadIdx.x;
    const int PN = P * N;

    const float Ah = gload(A + hd);  // issued with the first loads, off the dependency chain
    // the path indices and the parents head the only dependent chain (indices,
    // then the path's rows), so they leave first, the accepted row without
    // waiting for its length
    const int len = accepted_len[b];
    int acc_i[NPT], par_i[NPT];
#pragma unroll
    for (int m = 0; m < NPT; ++m)
        acc_i[m] = Lmax > 0 ? accepted[(size_t)b * Lmax + min(tid + kBlock * m, Lmax - 1)] : 0;
    if (NPT == 1) {
        par_i[0] = load_parent(parent + (size_t)b * T, T);
    } else {
#pragma unroll
        for (int m = 0; m < NPT; ++m) par_i[m] = gload(parent + (size_t)b * T + min(tid + kBlock * m, T - 1));
    }
    // PRE: piece tid of every node's x rows and of every node's B rows, and
    // node tid's dt, ahead of the state (waiting for them leaves the state in
    // flight); clamped, so every thread issues the same loads
    constexpr bool pre = PRE && sizeof(TIO) == 2 && VEC;  // the launch checks the sizes
    const int px = P / 8, pb = N / 8;
    uint4 rx = make_uint4(0, 0, 0, 0), rb = rx;
    uint32_t rdt = 0;
    if (pre) {
        const int ex = min(tid, T * px - 1), eb = min(tid, T * pb - 1);
        rx = gload((const uint4*)(x + (((size_t)b * T + ex / px) * H + hd) * P + 8 * (ex % px)));
        rb = gload((const uint4*)(Bm + (((size_t)b * T + eb / pb) * G + g) * N + 8 * (eb % pb)));
        rdt = gload((const uint16_t*)dt + ((size_t)b * T + min(tid, T - 1)) * H + hd);
    }
    // state chunk (written back only for a valid item)
    float* hb = h + ((size_t)b * H + hd) * PN;
    const int e0 = chunk * (kBlock * kVec * 4);
    float acc[kVec][4];
    int pe[kVec];
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
        pe[v] = e0 + (v * kBlock + tid) * 4;
        if (VEC) {
            // unconditional (clamped) loads, so that waits for the earlier
            // index loads can leave these in flight
            float4 t = gload_nt((const float4*)(hb + min(pe[v], PN - 4)));
            if (pe[v] >= PN) t = make_float4(0.f, 0.f, 0.f, 0.f);
            acc[v][0] = t.x;
            acc[v][1] = t.y;
            acc[v][2] = t.z;
            acc[v][3] = t.w;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[v][c] = (pe[v] + c < PN) ? gload(hb + pe[v] + c) : 0.f;
        }
    }

    // tree and path indices (one round trip, with the state chunk)
    // a valid path steps from parent to child, so its indices increase and
    // len <= T (this also keeps every path index inside s_path)
    const bool len_ok = len >= 0 && len <= Lmax && len <= T;
#pragma unroll
    for (int m = 0; m < NPT; ++m)
        if (len_ok && tid + kBlock * m < len) s_path[tid + kBlock * m] = acc_i[m];
    if (pre && tid < T) s_pos[tid] = -1;
    // LDS-only barriers from here on: the state chunk stays in flight while the
    // tree and path are checked and the path rows are requested
    int st;
    if (NPT == 1) {
        st = check_tree_lds<kBlock>(par_i[0], T, s_par, s_red);  // barrier: s_path visible too
    } else {
        int bad_root = 0, bad_par = 0;
#pragma unroll
        for (int m = 0; m < NPT; ++m) {
            const int i = tid + kBlock * m, p = par_i[m];
            if (i < T) {
                s_par[i] = p;
                if (i == 0)
                    bad_root = p != -1;
                else
                    bad_par |= p < 0 || p >= i;
            }
        }
        st = 0;
        if (lds_sync_or<kBlock>(bad_root | bad_par, s_red)) {  // barrier: s_par, s_path visible
            st = lds_sync_or<kBlock>(bad_root, s_red) ? kStBadRoot : 0;
            st |= lds_sync_or<kBlock>(bad_par, s_red) ? kStBadParent : 0;
        }
    }
    int bad_path = 0;
    if (!st) {
        if (!len_ok) {
            bad_path = 1;
        } else {
#pragma unroll
            for (int m = 0; m < NPT; ++m) {
                const int k = tid + kBlock * m;
                if (k < len) {
                    const int node = s_path[k];
                    if (k == 0)
                        bad_path |= node != 0;
                    else
                        bad_path |= node < 0 || node >= T || s_par[node] != s_path[k - 1];
                    if (pre && node >= 0 && node < T) s_pos[node] = k;  // used only for a valid path
                }
            }
        }
    }
    if (lds_sync_or<kBlock>(bad_path, s_red)) st |= kStBadPath;
    if (layer == 0 && hd == 0 && chunk == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st || len == 0) return;

    // path rows, one round trip per chunk of kPathChunk entries: dt of every
    // entry, raw x rows and B rows; the decay weights are formed once all dt are in
    auto stage_rows = [&](int k0, int kn) {
        if (sizeof(TIO) == 2 && P % 8 == 0 && N % 8 == 0) {
            // bf16 rows in 16-byte pieces: one x piece and one B piece per thread
            // and pass, both loads issued before either is used (one pass for
            // head_dim 64 and d_state 128)
            const int px = P / 8, pb = N / 8;
            const int nx = kn * px, nb = kn * pb;
            for (int e = tid; e < max(nx, nb); e += kBlock) {
                uint4 vx = make_uint4(0, 0, 0, 0), vb = vx;
                if (e < nx) {
                    const int k = e / px, c = e - k * px;
                    vx = gload((const uint4*)(x + (((size_t)b * T + s_path[k0 + k]) * H + hd) * P + 8 * c));
                }
                if (e < nb) {
                    const int k = e / pb, c = e - k * pb;
                    vb = gload((const uint4*)(Bm + (((size_t)b * T + s_path[k0 + k]) * G + g) * N + 8 * c));
                }
                if (e < nx) put8(s_wx + 8 * e, vx);  // piece e: row e / px, columns 8 (e % px) ..
                if (e < nb) put8(s_B + 8 * e, vb);
            }
            return;
        }
        for (int e = tid; e < kn * P; e += kBlock) {
            const int k = e / P, p = e - k * P;
            s_wx[k * P + p] = Elem<TIO>::ld(x, (((size_t)b * T + s_path[k0 + k]) * H + hd) * P + p);
        }
        for (int e = tid; e < kn * N; e += kBlock) {
            const int k = e / N, n = e - k * N;
            s_B[k * N + n] = Elem<TIO>::ld(Bm, (((size_t)b * T + s_path[k0 + k]) * G + g) * N + n);
        }
    };
    for (int k0 = 0; k0 < len; k0 += kPathChunk) {
        const int kn = min(kPathChunk, len - k0);
        if (k0 > 0) lds_barrier();  // previous chunk consumed
        if (pre) {
            // len <= Lmax <= kPathChunk: one chunk; the path's rows out of the
            // preloaded pieces, at their path positions
            if (tid < T && s_pos[tid] >= 0) s_w[s_pos[tid]] = bf16_bits_to_f32(rdt);
            if (tid < T * px && s_pos[tid / px] >= 0) put8(s_wx + 8 * (s_pos[tid / px] * px + tid % px), rx);
            if (tid < T * pb && s_pos[tid / pb] >= 0) put8(s_B + 8 * (s_pos[tid / pb] * pb + tid % pb), rb);
        } else {
            if (k0 == 0)
#pragma unroll
                for (int m = 0; m < NPT; ++m)
                    if (tid + kBlock * m < len)
                        s_w[tid + kBlock * m] = Elem<TIO>::ld(dt, ((size_t)b * T + s_path[tid + kBlock * m]) * H + hd);
            stage_rows(k0, kn);
        }
        lds_barrier();
        if (k0 == 0) {
            // decay weights along the path: w_k = exp(c_{k+1}) dt_{j_k}, w0 = exp(c_0)
            if (tid == 0) {
                float c = 0.f;
                for (int k = len - 1; k >= 0; --k) {
                    const float dtk = s_w[k];
                    s_w[k] = expf(c) * dtk;
                    c += dtk * Ah;
                }
                s_w0 = expf(c);
            }
            lds_barrier();
            const float w0 = s_w0;
#pragma unroll
            for (int v = 0; v < kVec; ++v)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[v][c] *= w0;
        }
        // weight the staged x rows in place
        for (int e = tid; e < kn * P; e += kBlock) s_wx[e] *= s_w[k0 + e / P];
        lds_barrier();
        if (VEC && (kBlock * 4) % N == 0 && pe[kVec - 1] < PN) {
            // every float4 of this thread covers the same columns n .. n+3 of
            // its own row p_v: one B read per path entry serves all of them,
            // and the reads of an entry leave together
            const int n = pe[0] % N;
            int pv[kVec];
#pragma unroll
            for (int v = 0; v < kVec; ++v) pv[v] = pe[v] / N;
#pragma unroll 1
            for (int k = 0; k < kn; ++k) {
                const float4 bb = *(const float4*)(s_B + k * N + n);
                float wx[kVec];
#pragma unroll
                for (int v = 0; v < kVec; ++v) wx[v] = s_wx[k * P + pv[v]];
#pragma unroll
                for (int v = 0; v < kVec; ++v) {
                    acc[v][0] += wx[v] * bb.x;
                    acc[v][1] += wx[v] * bb.y;
                    acc[v][2] += wx[v] * bb.z;
                    acc[v][3] += wx[v] * bb.w;
                }
            }
            continue;
        }
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
            if (VEC) {
                if (pe[v] >= PN) continue;
                const int p = pe[v] / N, n = pe[v] - p * N;  // 4 consecutive n of one row p
                float a0 = acc[v][0], a1 = acc[v][1], a2 = acc[v][2], a3 = acc[v][3];
                for (int k = 0; k < kn; ++k) {
                    const float wx = s_wx[k * P + p];
                    const float4 bb = *(const float4*)(s_B + k * N + n);
                    a0 += wx * bb.x;
                    a1 += wx * bb.y;
                    a2 += wx * bb.z;
                    a3 += wx * bb.w;
                }
                acc[v][0] = a0;
                acc[v][1] = a1;
                acc[v][2] = a2;
                acc[v][3] = a3;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int e = pe[v] + c;
                    if (e >= PN) continue;
                    const int p = e / N, n = e - p * N;
                    float a = acc[v][c];
                    for (int k = 0; k < kn; ++k) a += s_wx[k * P + p] * s_B[k * N + n];
                    acc[v][c] = a;
                }
            }
        }
    }
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
        if (VEC) {
            if (pe[v] < PN)
                gstore_nt((float4*)(hb + pe[v]), make_float4(acc[v][0], acc[v][1], acc[v][2], acc[v][3]));
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (pe[v] + c < PN) gstore(hb + pe[v] + c, acc[v][c]);
        }
    }
}

template <int NPT>
static hipError_t launch_commit_npt(const CommitArgs& a, bool bf16, hipStream_t stream) {
    const int per_wg = kBlock * kVec * 4;
    const int chunks = (a.P * a.N + per_wg - 1) / per_wg;
    const int BH = a.batch * a.H;
    dim3 grid((unsigned)((size_t)a.n_layers * BH * chunks));
    const size_t lds = sizeof(float) * kPathChunk * (size_t)(a.P + a.N);
    const bool vec = (a.N % 4) == 0;
    // one piece of every node's x and B rows per thread, the path in one chunk
    const bool pre = NPT == 1 && bf16 && vec && a.P % 8 == 0 && a.N % 8 == 0 && a.T * (a.P / 8) <= kBlock &&
                     a.T * (a.N / 8) <= kBlock && 4 * a.T <= a.N && a.Lmax <= kPathChunk;
#define TSV_COMMIT(TIO, V, PR)                                                               \
    hipLaunchKernelGGL((commit_kernel<TIO, V, PR && NPT == 1, NPT>), grid, dim3(kBlock), lds, stream, \
                       (const TIO*)a.x, (const TIO*)a.dt, a.A, (const TIO*)a.B, a.h, a.layers, \
                       a.parent, a.accepted, a.accepted_len, a.tree_status, BH, a.T, a.H, a.P, \
                       a.N, a.G, a.Lmax, chunks)
    if (bf16) {
        if (pre) TSV_COMMIT(uint16_t, true, true);
        else if (vec) TSV_COMMIT(uint16_t, true, false);
        else TSV_COMMIT(uint16_t, false, false);
    } else {
        if (vec) TSV_COMMIT(float, true, false);
        else TSV_COMMIT(float, false, false);
    }
#undef TSV_COMMIT
    return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, bool bf16, hipStream_t stream) {
    return a.T <= kMaxNodes ? launch_commit_npt<1>(a, bf16, stream) : launch_commit_npt<4>(a, bf16, stream);
}

}  // namespace tsv
