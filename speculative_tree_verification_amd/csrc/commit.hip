// commit.hip -- activation replay: rebuild, in place, the state at the end of
// the accepted root path ("STree: Speculative Tree Decoding for Hybrid State
// Space Models", atlas.scime.ai summary, section "Approach": "activation replay
// for state backtracking"). For the path j_0 = 0, ..., j_{L-1} = l:
//   H' = exp(c_0) h0 + sum_k exp(c_{k+1}) dt_{j_k} x_{j_k} (outer) B_{j_k},
// with c_k = sum_{m >= k} dt_{j_m} A the log decay from after token j_{k-1}
// to the end of the path (suffix sums, so no cancellation).
//
// Work-group = (batch item, head, chunk of the P x N state). Every work-group
// re-validates the tree and the path (bit-exact integer checks) and leaves
// h0 untouched when either is bad. The state is streamed once: each element
// is read and written by the same thread (rank-L update in registers).
#include "common.hpp"
#include "launch.hpp"

namespace tsv {

constexpr int kPathChunk = 16;  // path entries staged in LDS at a time
constexpr int kMaxDim = 256;    // P, N limit of the staging buffers
constexpr int kVec = 4;         // float4 per thread per chunk

template <typename TIO, bool VEC>
__global__ __launch_bounds__(kBlock) void commit_kernel(
    const TIO* __restrict__ x, const TIO* __restrict__ dt, const float* __restrict__ A,
    const TIO* __restrict__ Bm, float* __restrict__ h, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ accepted, const int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ tree_status, int T, int H, int P, int N, int G, int Lmax,
    int chunks) {
    __shared__ int s_par[kMaxNodes];
    __shared__ int s_path[kMaxNodes];
    __shared__ float s_w[kMaxNodes];
    __shared__ float s_dtp[kMaxNodes];
    __shared__ float s_wx[kPathChunk][kMaxDim];
    __shared__ float s_B[kPathChunk][kMaxDim];
    __shared__ float s_w0;

    const int chunk = blockIdx.x % chunks;
    const int bh = blockIdx.x / chunks;
    const int b = bh / H;
    const int hd = bh % H;
    const int g = hd / (H / G);
    const int tid = threadIdx.x;

    int st = load_tree(parent + (size_t)b * T, T, s_par);
    const int len = accepted_len[b];
    // the path is checked only on a valid tree (its parent links are meaningful)
    int bad_path = !st && (len < 0 || len > Lmax);
    if (!st && !bad_path) {
        for (int k = tid; k < len; k += kBlock) {
            const int node = accepted[(size_t)b * Lmax + k];
            s_path[k] = node;
            if (node >= 0 && node < T)
                s_dtp[k] = Elem<TIO>::ld(dt, ((size_t)b * T + node) * H + hd);
            if (k == 0) {
                if (node != 0) bad_path = 1;
            } else {
                const int prev = accepted[(size_t)b * Lmax + k - 1];
                if (node < 0 || node >= T || s_par[node] != prev) bad_path = 1;
            }
        }
    }
    if (__syncthreads_or(bad_path)) st |= kStBadPath;
    if (hd == 0 && chunk == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st || len == 0) return;

    const float Ah = A[hd];
    if (tid == 0) {
        // suffix sums along the path: weight of token k is exp(decay after it) * dt
        float c = 0.f;
        for (int k = len - 1; k >= 0; --k) {
            const float dtk = s_dtp[k];
            s_w[k] = expf(c) * dtk;
            c += dtk * Ah;
        }
        s_w0 = expf(c);
    }
    __syncthreads();
    const float w0 = s_w0;

    float* hb = h + ((size_t)b * H + hd) * P * N;
    const int per_chunk = kBlock * kVec * 4;
    const int e0 = chunk * per_chunk;
    float acc[kVec][4];
    int pe[kVec];
    bool live[kVec];
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
        pe[v] = e0 + (v * kBlock + tid) * 4;
        live[v] = pe[v] < P * N;
        if (VEC) {
            float4 t = live[v] ? *(const float4*)(hb + pe[v]) : make_float4(0.f, 0.f, 0.f, 0.f);
            acc[v][0] = w0 * t.x;
            acc[v][1] = w0 * t.y;
            acc[v][2] = w0 * t.z;
            acc[v][3] = w0 * t.w;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[v][c] = (pe[v] + c < P * N) ? w0 * hb[pe[v] + c] : 0.f;
        }
    }
    for (int k0 = 0; k0 < len; k0 += kPathChunk) {
        const int kn = min(kPathChunk, len - k0);
        __syncthreads();
        for (int e = tid; e < kn * P; e += kBlock) {
            const int k = e / P, p = e % P;
            s_wx[k][p] = s_w[k0 + k] *
                         Elem<TIO>::ld(x, (((size_t)b * T + s_path[k0 + k]) * H + hd) * P + p);
        }
        for (int e = tid; e < kn * N; e += kBlock) {
            const int k = e / N, n = e % N;
            s_B[k][n] = Elem<TIO>::ld(Bm, (((size_t)b * T + s_path[k0 + k]) * G + g) * N + n);
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int e = pe[v] + c;
                if (e >= P * N) continue;
                const int p = e / N, n = e % N;
                float a = acc[v][c];
                for (int k = 0; k < kn; ++k) a += s_wx[k][p] * s_B[k][n];
                acc[v][c] = a;
            }
        }
    }
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
        if (VEC) {
            if (live[v])
                *(float4*)(hb + pe[v]) = make_float4(acc[v][0], acc[v][1], acc[v][2], acc[v][3]);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (pe[v] + c < P * N) hb[pe[v] + c] = acc[v][c];
        }
    }
}

hipError_t launch_commit(const CommitArgs& a, bool bf16, hipStream_t stream) {
    const int per_chunk = kBlock * kVec * 4;
    const int chunks = (a.P * a.N + per_chunk - 1) / per_chunk;
    dim3 grid((unsigned)(a.batch * a.H * chunks));
    const bool vec = (a.N % 4) == 0;
#define TSV_COMMIT(TIO, V)                                                                   \
    hipLaunchKernelGGL((commit_kernel<TIO, V>), grid, dim3(kBlock), 0, stream,               \
                       (const TIO*)a.x, (const TIO*)a.dt, a.A, (const TIO*)a.B, a.h, a.parent, \
                       a.accepted, a.accepted_len, a.tree_status, a.T, a.H, a.P, a.N, a.G,   \
                       a.Lmax, chunks)
    if (bf16) {
        if (vec) TSV_COMMIT(uint16_t, true);
        else TSV_COMMIT(uint16_t, false);
    } else {
        if (vec) TSV_COMMIT(float, true);
        else TSV_COMMIT(float, false);
    }
#undef TSV_COMMIT
    return hipGetLastError();
}

}  // namespace tsv
