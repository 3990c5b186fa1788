// accept_stochastic.hip -- stochastic acceptance of a verified draft tree:
// multi-step speculative sampling with siblings drawn without replacement
// ("STree: Speculative Tree Decoding for Hybrid State-Space Models",
// atlas.scime.ai summary, measured-effects table: multi-step speculative
// sampling as the acceptance rule; "TreeSpark: Adaptive Draft Trees Accelerate
// Speculative Decoding by 8-14%", section on the lossless guarantee: siblings
// sampled without replacement, rejected tokens resampled from the residual of
// target and draft).
//
// The walk starts at the root with residual r = p (the target distribution
// after the current node u). The children of u are tested in index order; the
// k-th child's token t was drawn from d = q / m, q the draft distribution of u
// with the earlier children's tokens removed and m = 1 - (their draft mass).
// It is accepted when u_node * d(t) < r(t). A rejection replaces r by
// max(r - d, 0) / Z (Z its mass; r is kept when Z is 0). An accepted child
// becomes u; when every child is rejected the next token is drawn from r by
// inverse CDF with u_final.
//
// Closed form. Before any removal d = q / m on every token, and a rejected
// token t always has r(t) < d(t) (otherwise u * d(t) < r(t) for every u < 1),
// so its residual becomes 0 and stays 0. Hence on every token not yet removed
// at u the residual is max(a p(x) - b q(x), 0) for two scalars: a = 1, b = 0
// at the start, and a rejection with mass m maps (a, b) to
// (a / Z, (b + 1 / m) / Z). Removed tokens keep an explicit value (a short
// list in LDS, divided by Z at each rejection), which covers a residual of no
// mass and repeated sibling tokens exactly as the step-by-step rule. So a
// rejection costs one pass over the vocabulary (the mass Z), and no residual
// vector is ever stored: the kernel needs no workspace.
//
// One 1024-thread work-group per item. Decisions are taken in fp64; every
// thread carries the same scalars (a, b, m, the walk's node), and the passes
// split the vocabulary into 16 contiguous wave segments. Each node's test
// inputs -- p(u)[t], q(u)[t] for its own token t under its parent u, and its
// uniform -- are gathered into LDS before the walk, so a test never waits for
// memory. The final draw takes the segment masses from the last rejection's
// pass (one more pass only at a node without children), picks the segment by
// a prefix over the 16, and walks that segment in 256-token chunks with a
// wave prefix sum.
#include "common.hpp"
#include "launch.hpp"

namespace tsv {

namespace {

constexpr int kSNT = 1024;               // threads per item
constexpr int kSWaves = kSNT / kWave;    // vocabulary segments
constexpr int kSMaxNodes = 1024;

__device__ __forceinline__ double resid(double a, double b, float p, float q) {
    return fmax(a * (double)p - b * (double)q, 0.0);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// four consecutive residual values starting at x (x a multiple of 4 when VEC);
// tokens at or past `end` give 0
template <bool VEC>
__device__ __forceinline__ void load4(const float* __restrict__ pr, const float* __restrict__ qr,
                                      int x, int end, bool useq, double a, double b, double r[4]) {
    if (VEC) {
        if (x < end) {
            const float4 pv = *(const float4*)(pr + x);
            float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (useq) qv = *(const float4*)(qr + x);
            r[0] = resid(a, b, pv.x, qv.x);
            r[1] = resid(a, b, pv.y, qv.y);
            r[2] = resid(a, b, pv.z, qv.z);
            r[3] = resid(a, b, pv.w, qv.w);
        } else {
            r[0] = r[1] = r[2] = r[3] = 0.0;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int xj = x + j;
            r[j] = xj < end ? resid(a, b, pr[xj], useq ? qr[xj] : 0.f) : 0.0;
        }
    }
}

// this lane's part of the residual mass of segment [s0, s1): chunks of 256
// tokens, 4 consecutive tokens per lane
template <bool VEC>
__device__ __forceinline__ double lane_mass(const float* __restrict__ pr, const float* __restrict__ qr,
                                            int s0, int s1, bool useq, double a, double b, int lane) {
    double acc = 0.0;
    int x = s0 + 4 * lane;
    for (; x + 3 * 4 * kWave < s1; x += 4 * 4 * kWave) {  // four chunks in flight
        double r[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) load4<VEC>(pr, qr, x + k * 4 * kWave, s1, useq, a, b, r[k]);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc += (r[k][0] + r[k][1]) + (r[k][2] + r[k][3]);
    }
    for (; x < s1; x += 4 * kWave) {
        double r[4];
        load4<VEC>(pr, qr, x, s1, useq, a, b, r);
        acc += (r[0] + r[1]) + (r[2] + r[3]);
    }
    return acc;
}

template <bool VEC>
__global__ __launch_bounds__(kSNT) void accept_stochastic_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ draft,
    const float* __restrict__ p_target, const float* __restrict__ q_draft,
    const float* __restrict__ u_node, const float* __restrict__ u_final, int T, int V, int Lmax,
    int32_t* __restrict__ accepted, int32_t* __restrict__ accepted_len, int32_t* __restrict__ next_token,
    int32_t* __restrict__ tree_status) {
    __shared__ int s_par[kSMaxNodes];
    __shared__ int s_tok[kSMaxNodes];
    __shared__ float s_pt[kSMaxNodes];   // p(parent)[own token]
    __shared__ float s_qt[kSMaxNodes];   // q(parent)[own token]
    __shared__ float s_un[kSMaxNodes];   // own uniform
    __shared__ int s_etok[kSMaxNodes];   // tokens removed at the current node
    __shared__ double s_eval[kSMaxNodes];  // their residual values
    __shared__ int s_path[kSMaxNodes];
    __shared__ uint64_t s_ball[2][kSWaves];
    __shared__ double s_seg[kSWaves];
    __shared__ int s_pick;

    const int bi = blockIdx.x;
    const int i = threadIdx.x;
    const int lane = i & (kWave - 1);
    const int w = i >> 6;
    const size_t row0 = (size_t)bi * T;

    // ---- set-up: tree check, token range, each node's test inputs
    const int p = load_parent(parent + row0, T);
    const int tok = i < T ? draft[row0 + i] : 0;
    const bool bad_tok = i >= 1 && i < T && (tok < 0 || tok >= V);
    float pt = 0.f, qt = 0.f, un = 0.f;
    if (i >= 1 && i < T && !bad_tok && p >= 0 && p < i) {
        const size_t prow = (row0 + p) * (size_t)V;
        pt = p_target[prow + tok];
        qt = q_draft[prow + tok];
        un = u_node[row0 + i];
    }
    int st = check_tree(p, T, s_par);
    if (__syncthreads_or(bad_tok)) st |= kStBadToken;
    if (i == 0 && tree_status) tree_status[bi] = st;
    if (st) return;
    if (i < T) {
        s_tok[i] = tok;
        s_pt[i] = pt;
        s_qt[i] = qt;
        s_un[i] = un;
    }
    if (i == 0) s_path[0] = 0;
    const int seg = ((V + 4 * kSWaves - 1) / (4 * kSWaves)) * 4;
    const int s0 = min(w * seg, V), s1 = min(s0 + seg, V);

    // ---- the walk (every thread holds the same scalars)
    int u = 0, len = 1, next = -1, par_buf = 0;
    for (;;) {
        // children of u in index order: one ballot word per wave
        const uint64_t bits = __ballot(i < T && i > 0 && s_par[i] == u);
        if (lane == 0) s_ball[par_buf][w] = bits;
        __syncthreads();
        const float* pr = p_target + (row0 + u) * (size_t)V;
        const float* qr = q_draft + (row0 + u) * (size_t)V;
        double a = 1.0, b = 0.0, removed = 0.0;
        int ne = 0, child = -1;
        // the last rejection's pass: its segment masses serve the final draw
        double last_z = 0.0, last_a = 0.0, last_b2 = 0.0;
        int last_ne = 0;
        for (int cw = 0; cw < kSWaves && child < 0; ++cw) {
            uint64_t m = s_ball[par_buf][cw];
            while (m && child < 0) {
                const int c = cw * kWave + __builtin_ctzll(m);
                m &= m - 1;
                const int t = s_tok[c];
                int dup = -1;
                for (int j = 0; j < ne; ++j)
                    if (s_etok[j] == t) dup = j;
                const double mass = 1.0 - removed;
                const double qt_d = (double)s_qt[c];
                const double dt = (dup >= 0 || !(mass > 0.0)) ? 0.0 : qt_d / mass;
                const double rt = dup >= 0 ? s_eval[dup] : resid(a, b, s_pt[c], s_qt[c]);
                if ((double)s_un[c] * dt < rt) {
                    child = c;
                    break;
                }
                // rejected: residual mass Z of max(r - d, 0), r moves to it
                const double b2 = mass > 0.0 ? b + 1.0 / mass : b;
                const double part = wave_sum(lane_mass<VEC>(pr, qr, s0, s1, b2 != 0.0, a, b2, lane));
                if (lane == 0) s_seg[w] = part;
                __syncthreads();
                double z = 0.0;
#pragma unroll
                for (int k = 0; k < kSWaves; ++k) z += s_seg[k];
                for (int j = 0; j < ne; ++j) {
                    const int e = s_etok[j];
                    z += s_eval[j] - resid(a, b2, pr[e], qr[e]);
                }
                const double tval = dup >= 0 ? 0.0 : resid(a, b2, s_pt[c], s_qt[c]);
                last_z = z;
                last_a = a;
                last_b2 = b2;
                last_ne = ne;
                __syncthreads();  // every thread has read s_seg and the list
                if (z > 0.0) {
                    a = a / z;
                    b = b2 / z;
                    if (i < ne) s_eval[i] = s_eval[i] / z;
                }
                if (dup < 0) {
                    if (i == 0) {
                        s_etok[ne] = t;
                        s_eval[ne] = z > 0.0 ? tval / z : resid(a, b, s_pt[c], s_qt[c]);
                    }
                    ++ne;
                    removed += qt_d;
                }
                __syncthreads();
            }
        }
        par_buf ^= 1;
        if (child >= 0) {
            if (len == Lmax) {
                next = s_tok[child];
                break;
            }
            if (i == 0) s_path[len] = child;
            ++len;
            u = child;
            continue;
        }

        // ---- no child accepted: draw the next token from the residual. Its
        // segment masses: after a rejection of positive mass, that pass's
        // masses divided by it (the residual is that pass's values over Z on
        // every token but the earlier removed ones); otherwise one more pass.
        const bool useq = b != 0.0;
        if (last_z > 0.0) {
            if (i == 0) {
                for (int k = 0; k < kSWaves; ++k) s_seg[k] = s_seg[k] / last_z;
                for (int j = 0; j < last_ne; ++j) {
                    const int e = s_etok[j];
                    s_seg[e / seg] += s_eval[j] - resid(last_a, last_b2, pr[e], qr[e]) / last_z;
                }
                s_pick = -1;
            }
        } else {
            const double part = wave_sum(lane_mass<VEC>(pr, qr, s0, s1, useq, a, b, lane));
            if (lane == 0) s_seg[w] = part;
            __syncthreads();
            if (i == 0) {
                for (int j = 0; j < ne; ++j) {
                    const int e = s_etok[j];
                    s_seg[e / seg] += s_eval[j] - resid(a, b, pr[e], qr[e]);
                }
                s_pick = -1;
            }
        }
        __syncthreads();
        double total = 0.0;
        double before = 0.0;
        int wsel = -1;
        const double uf = (double)u_final[bi];
        {
            double run = 0.0;
            for (int k = 0; k < kSWaves; ++k) run += s_seg[k];
            total = run;
            const double thr = uf * total;
            run = 0.0;
            for (int k = 0; k < kSWaves; ++k) {
                const double nr = run + s_seg[k];
                if (wsel < 0 && nr > thr) {
                    wsel = k;
                    before = run;
                }
                run = nr;
            }
        }
        if (total > 0.0 && wsel >= 0 && w == wsel) {
            const double thr = uf * total;
            const int e0 = min(wsel * seg, V), e1 = min(e0 + seg, V);
            double base = before;
            int last_pos = -1, found = -1;
            for (int c0 = e0; c0 < e1 && found < 0; c0 += 4 * kWave) {
                const int x = c0 + 4 * lane;
                double r[4];
                load4<VEC>(pr, qr, x, e1, useq, a, b, r);
                for (int j = 0; j < ne; ++j) {
                    const int off = s_etok[j] - x;
                    const double v = s_eval[j];
                    r[0] = off == 0 ? v : r[0];
                    r[1] = off == 1 ? v : r[1];
                    r[2] = off == 2 ? v : r[2];
                    r[3] = off == 3 ? v : r[3];
                }
                const double ls = (r[0] + r[1]) + (r[2] + r[3]);
                const double incl = wave_incl_scan(ls, lane);
                double excl = __shfl_up(incl, 1, kWave);
                if (lane == 0) excl = 0.0;
                const double tot = __shfl(incl, kWave - 1, kWave);
                // last token with positive residual so far (fallback of the draw)
                int lp = -1;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (r[j] > 0.0) lp = x + j;
                const uint64_t any = __ballot(lp >= 0);
                if (any) last_pos = __shfl(lp, 63 - __builtin_clzll(any), kWave);
                if (base + tot > thr) {
                    const uint64_t hit = __ballot(base + incl > thr);
                    const int hl = hit ? __builtin_ctzll(hit) : kWave - 1;
                    int pick = -1;
                    if (lane == hl) {
                        double run = base + excl;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            run += r[j];
                            if (pick < 0 && run > thr) pick = x + j;
                        }
                        if (pick < 0) pick = lp;
                    }
                    found = __shfl(pick, hl, kWave);
                }
                base += tot;
            }
            if (lane == 0) s_pick = found >= 0 ? found : last_pos;
        }
        __syncthreads();
        next = s_pick;
        break;
    }

    __syncthreads();  // s_path complete
    int32_t* arow = accepted + (size_t)bi * Lmax;
    for (int k = i; k < Lmax; k += kSNT) arow[k] = k < len ? s_path[k] : -1;
    if (i == 0) {
        accepted_len[bi] = len;
        if (next_token) next_token[bi] = next;
    }
}

}  // namespace

hipError_t launch_accept_stochastic(int batch, int T, int V, const int32_t* parent, const int32_t* draft,
                                    const float* p_target, const float* q_draft, const float* u_node,
                                    const float* u_final, int Lmax, int32_t* accepted, int32_t* accepted_len,
                                    int32_t* next_token, int32_t* tree_status, hipStream_t stream) {
    const bool vec = V % 4 == 0 && ((uintptr_t)p_target % 16) == 0 && ((uintptr_t)q_draft % 16) == 0;
    if (vec)
        hipLaunchKernelGGL(accept_stochastic_kernel<true>, dim3(batch), dim3(kSNT), 0, stream, parent, draft,
                           p_target, q_draft, u_node, u_final, T, V, Lmax, accepted, accepted_len, next_token,
                           tree_status);
    else
        hipLaunchKernelGGL(accept_stochastic_kernel<false>, dim3(batch), dim3(kSNT), 0, stream, parent, draft,
                           p_target, q_draft, u_node, u_final, T, V, Lmax, accepted, accepted_len, next_token,
                           tree_status);
    return hipGetLastError();
}

}  // namespace tsv
