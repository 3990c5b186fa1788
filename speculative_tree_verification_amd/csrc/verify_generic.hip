// verify_generic.hip -- packed-tree verification of one SSD layer, plain fp32
// VALU form for any head_dim / d_state (<= 256) and both input dtypes.
//
// Method: "STree: Speculative Tree Decoding for Hybrid State Space Models"
// (atlas.scime.ai summary, section "Approach"). For node i with root path
// pi(i), log decays accumulated along the path (cum = L * (dt A)) give
//   y_i[p] = exp(cum_i) (h0 C_i)[p]
//          + sum_{j in pi(i)} (C_i . B_j) exp(cum_i - cum_j) dt_j x_j[p] + D x_i[p].
// cum_i - cum_j is summed directly along the walk from i up to j (no
// difference of two prefix sums), so no cancellation and no overflow from
// non-ancestor pairs, which are never visited.
//
// One work-group per (batch item, head); one thread per output element (i, p).
// This is the reference-grade GPU path (fp32 inputs, unusual shapes); the
// MFMA kernel covers the bf16 Mamba2 shapes.
#include "common.hpp"
#include "launch.hpp"

namespace tsv {

template <typename TIO>
__global__ __launch_bounds__(kBlock) void verify_generic_kernel(
    const TIO* __restrict__ x, const TIO* __restrict__ dt, const float* __restrict__ A,
    const TIO* __restrict__ Bm, const TIO* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ h0, const int32_t* __restrict__ parent, TIO* __restrict__ y,
    int32_t* __restrict__ tree_status, int T, int H, int P, int N, int G) {
    __shared__ int s_par[kMaxNodes];
    __shared__ float s_dt[kMaxNodes];

    const int b = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int g = h / (H / G);
    const int st = load_tree(parent + (size_t)b * T, T, s_par);
    if (h == 0 && threadIdx.x == 0 && tree_status) tree_status[b] = st;
    if (st) return;

    const float Ah = A[h];
    const float Dh = D[h];
    for (int i = threadIdx.x; i < T; i += kBlock)
        s_dt[i] = Elem<TIO>::ld(dt, ((size_t)b * T + i) * H + h);
    __syncthreads();

    const float* H0 = h0 + ((size_t)b * H + h) * P * N;
    for (int e = threadIdx.x; e < T * P; e += kBlock) {
        const int i = e / P;
        const int p = e % P;
        const TIO* Ci = Cm + (((size_t)b * T + i) * G + g) * N;
        float intra = 0.f;
        float s = 0.f;  // sum of dt*A over the nodes from i up to (excluding) j
        for (int j = i; j >= 0; j = s_par[j]) {
            const TIO* Bj = Bm + (((size_t)b * T + j) * G + g) * N;
            float gij = 0.f;
            for (int n = 0; n < N; ++n) gij += Elem<TIO>::ld(Ci, n) * Elem<TIO>::ld(Bj, n);
            const float dtj = s_dt[j];
            intra += gij * expf(s) * dtj * Elem<TIO>::ld(x, (((size_t)b * T + j) * H + h) * P + p);
            s += dtj * Ah;
        }
        float ch = 0.f;
        for (int n = 0; n < N; ++n) ch += Elem<TIO>::ld(Ci, n) * H0[(size_t)p * N + n];
        const size_t o = (((size_t)b * T + i) * H + h) * P + p;
        Elem<TIO>::st(y, o, expf(s) * ch + intra + Dh * Elem<TIO>::ld(x, o));
    }
}

hipError_t launch_verify_generic(const VerifyArgs& a, bool bf16, hipStream_t stream) {
    dim3 grid((unsigned)(a.batch * a.H));
    if (bf16) {
        hipLaunchKernelGGL(verify_generic_kernel<uint16_t>, grid, dim3(kBlock), 0, stream,
                           (const uint16_t*)a.x, (const uint16_t*)a.dt, a.A,
                           (const uint16_t*)a.B, (const uint16_t*)a.C, a.D, a.h0, a.parent,
                           (uint16_t*)a.y, a.tree_status, a.T, a.H, a.P, a.N, a.G);
    } else {
        hipLaunchKernelGGL(verify_generic_kernel<float>, grid, dim3(kBlock), 0, stream,
                           (const float*)a.x, (const float*)a.dt, a.A, (const float*)a.B,
                           (const float*)a.C, a.D, a.h0, a.parent, (float*)a.y, a.tree_status,
                           a.T, a.H, a.P, a.N, a.G);
    }
    return hipGetLastError();
}

}  // namespace tsv
