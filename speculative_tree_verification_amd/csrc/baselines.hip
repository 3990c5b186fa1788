// baselines.hip -- the two forms a packed-tree scan replaces, on the same
// inputs and layouts, so that their cost can be measured beside it.
//
// "STree: Speculative Tree Decoding for Hybrid State Space Models"
// (atlas.scime.ai summary): without a packed-tree scan an SSM unrolls the
// draft tree into repeated sequences, with extra states and memory (section
// "Problem"); the paper's baseline runs the unrolled tree through a fused
// selective scan (section "Experimental setup", times in "Key results"). The
// Bole and TreeWY abstracts (mlsanity and fugumt pages) name the other form:
// a full recurrent state materialised for every draft node.
//
//  * unrolled form: unroll_plan lists each item's leaves (nodes that are no
//    node's parent, by increasing index) and their root paths; unroll_gather
//    copies every path's rows of x, dt, B, C into sequence-major buffers and
//    gives every sequence its own copy of h0; seq_scan is an ordinary Mamba2
//    sequence scan over those sequences (it knows nothing of trees), writing
//    every position's output and each sequence's final state.
//  * snapshot form: snapshot_verify writes the state after every node to HBM
//    (each formed from its parent's stored state) and every node's output from
//    it; snapshot_commit copies the last accepted node's state into h0.
//
// Both are deliberately plain (fp32 VALU): their cost is the memory they
// materialise, which is what the packed form avoids.
#include "common.hpp"
#include "launch.hpp"

namespace tsv {

constexpr int kBaseThreads = 256;
constexpr int kTimeChunk = 16;     // time steps (or nodes) whose rows are staged in LDS at once
constexpr int kBaseMaxDim = 256;   // head_dim and d_state bound of the staging buffers
constexpr int kStBadCapacity = 8;  // plan: more leaves or a longer path than the buffers hold

// ---------------------------------------------------------------- plan
template <int NT>
__global__ __launch_bounds__(NT) void unroll_plan_kernel(const int32_t* __restrict__ parent, int T,
                                                         int Lcap, int S, int32_t* __restrict__ seq_nodes,
                                                         int32_t* __restrict__ seq_len,
                                                         int32_t* __restrict__ n_leaves,
                                                         int32_t* __restrict__ tree_status) {
    __shared__ int s_par[NT];
    __shared__ int s_child[NT];
    __shared__ int s_nxt[NT];
    __shared__ int s_dep[NT];
    __shared__ int s_scan[NT / kWave];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    int32_t* rows = seq_nodes + (size_t)b * Lcap * S;
    int32_t* lens = seq_len + (size_t)b * Lcap;
    const int par = load_parent(parent + (size_t)b * T, T);
    int st = check_tree(par, T, s_par);
    int leaf = 0, dep = 0, rank = 0, nl = 0;
    if (!st) {
        if (tid < T) s_child[tid] = 0;
        __syncthreads();
        if (tid > 0 && tid < T) s_child[par] = 1;
        __syncthreads();
        leaf = tid < T && !s_child[tid];
        dep = tree_depth(s_par, T, s_nxt, s_dep);
        rank = block_exclusive_scan<NT>(leaf, s_scan, &nl);
        if (__syncthreads_or(nl > Lcap || (leaf && dep + 1 > S))) st = kStBadCapacity;
    }
    if (tid == 0) {
        if (tree_status) tree_status[b] = st;
        n_leaves[b] = st ? 0 : nl;
    }
    if (st) nl = 0;
    // every slot past the item's leaves (all of them for an invalid item) is empty
    for (int e = nl * S + tid; e < Lcap * S; e += NT) rows[e] = -1;
    for (int l = nl + tid; l < Lcap; l += NT) lens[l] = 0;
    if (!st && leaf) {
        int32_t* row = rows + (size_t)rank * S;
        int j = tid;
        for (int k = dep; k >= 0; --k) {
            row[k] = j;
            j = s_par[j];
        }
        for (int k = dep + 1; k < S; ++k) row[k] = -1;
        lens[rank] = dep + 1;
    }
}

// ---------------------------------------------------------------- gather
// copy n elements of 2 or 4 bytes, 16 bytes at a time where both ends allow
template <typename E>
__device__ __forceinline__ void copy_elems(E* __restrict__ dst, const E* __restrict__ src, int n) {
    const bool vec = ((((uintptr_t)dst) | ((uintptr_t)src)) & 15) == 0 && (n * (int)sizeof(E)) % 16 == 0;
    if (vec) {
        const int nv = n * (int)sizeof(E) / 16;
        int i = threadIdx.x;
        for (; i + 3 * kBaseThreads < nv; i += 4 * kBaseThreads) {  // four loads in flight per thread
            uint4 t[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) t[u] = gload((const uint4*)src + i + u * kBaseThreads);
#pragma unroll
            for (int u = 0; u < 4; ++u) gstore((uint4*)dst + i + u * kBaseThreads, t[u]);
        }
        for (; i < nv; i += kBaseThreads) gstore((uint4*)dst + i, gload((const uint4*)src + i));
    } else {
        for (int i = threadIdx.x; i < n; i += kBaseThreads) gstore(dst + i, gload(src + i));
    }
}

// blocks [0, nseq S): one (sequence, position) row each; blocks [nseq S,
// nseq S + nseq H): one (sequence, head) copy of h0 each. Slots whose length
// or node index is out of range are skipped.
template <typename TIO>
__global__ __launch_bounds__(kBaseThreads) void unroll_gather_kernel(
    const TIO* __restrict__ x, const TIO* __restrict__ dt, const TIO* __restrict__ Bm,
    const TIO* __restrict__ Cm, const float* __restrict__ h0, const int32_t* __restrict__ seq_nodes,
    const int32_t* __restrict__ seq_len, int T, int H, int P, int N, int G, int Lcap, int S, int nseq,
    TIO* __restrict__ x_u, TIO* __restrict__ dt_u, TIO* __restrict__ B_u, TIO* __restrict__ C_u,
    float* __restrict__ h0_u) {
    const long blk = blockIdx.x;
    const long nrow = (long)nseq * S;
    if (blk < nrow) {
        const int seq = (int)(blk / S), s = (int)(blk % S);
        const int b = seq / Lcap;
        const int len = seq_len[seq];
        if (len < 0 || len > S || s >= len) return;
        const int node = seq_nodes[(size_t)seq * S + s];
        if (node < 0 || node >= T) return;
        const size_t src_row = (size_t)b * T + node, dst_row = (size_t)seq * S + s;
        copy_elems(x_u + dst_row * H * P, x + src_row * H * P, H * P);
        copy_elems(dt_u + dst_row * H, dt + src_row * H, H);
        copy_elems(B_u + dst_row * G * N, Bm + src_row * G * N, G * N);
        copy_elems(C_u + dst_row * G * N, Cm + src_row * G * N, G * N);
    } else {
        const long k = blk - nrow;
        const int seq = (int)(k / H), h = (int)(k % H);
        const int len = seq_len[seq];
        if (len <= 0 || len > S) return;
        const int b = seq / Lcap;
        copy_elems(h0_u + ((size_t)seq * H + h) * P * N, h0 + ((size_t)b * H + h) * P * N, P * N);
    }
}

// ---------------------------------------------------------------- rows staged in LDS
// kTimeChunk rows of x, y (head_dim each), B, C (d_state each) and dt, in the
// launch's dynamic LDS, sized to the shape so that several work-groups share a
// compute unit.
struct RowStage {
    float* xs;
    float* ys;
    float* Bs;
    float* Cs;
    float* dts;
    int P, N;
    __device__ __forceinline__ RowStage(float* base, int P_, int N_) : P(P_), N(N_) {
        xs = base;
        ys = xs + kTimeChunk * P;
        Bs = ys + kTimeChunk * P;
        Cs = Bs + kTimeChunk * N;
        dts = Cs + kTimeChunk * N;
    }
    __device__ __forceinline__ float* x(int t) { return xs + t * P; }
    __device__ __forceinline__ float* y(int t) { return ys + t * P; }
    __device__ __forceinline__ float* B(int t) { return Bs + t * N; }
    __device__ __forceinline__ float* C(int t) { return Cs + t * N; }
};
static size_t row_stage_bytes(int P, int N) { return sizeof(float) * ((size_t)kTimeChunk * (2 * P + 2 * N) + kTimeChunk); }

// ---------------------------------------------------------------- state slices
// Thread tid owns the KE consecutive state elements tid*KE .. tid*KE+KE-1 of
// the P x N state (row-major, n fastest), so its elements sit in one or a few
// rows and its part of y_t[p] = sum_n H[p][n] C_t[n] is summed in registers
// and added to the row's LDS total once per row it touches.
template <int KE>
struct StateSlice {
    float v[KE];
    int e0, p0, n0;  // first element, its row and column
    __device__ __forceinline__ void init(int PN, int N) {
        e0 = threadIdx.x * KE;
        p0 = e0 / N;
        n0 = e0 - p0 * N;
    }
    __device__ __forceinline__ void load(const float* __restrict__ src, int PN) {
        if ((KE % 4) == 0 && e0 + KE <= PN && (PN % 4) == 0) {
#pragma unroll
            for (int k = 0; k < KE; k += 4) {
                const float4 t = gload((const float4*)(src + e0 + k));
                v[k] = t.x;
                v[k + 1] = t.y;
                v[k + 2] = t.z;
                v[k + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < KE; ++k) v[k] = e0 + k < PN ? gload(src + e0 + k) : 0.f;
        }
    }
    __device__ __forceinline__ void store(float* __restrict__ dst, int PN) const {
        if ((KE % 4) == 0 && e0 + KE <= PN && (PN % 4) == 0) {
#pragma unroll
            for (int k = 0; k < KE; k += 4) gstore((float4*)(dst + e0 + k), make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]));
        } else {
#pragma unroll
            for (int k = 0; k < KE; ++k)
                if (e0 + k < PN) gstore(dst + e0 + k, v[k]);
        }
    }
    // one step of the recurrence from `src` (this thread's elements of the
    // previous state), adding this thread's part of y = H C to yrow
    __device__ __forceinline__ void step(const float (&src)[KE], float a, float d, const float* xr,
                                         const float* Br, const float* Cr, float* yrow, int PN, int N) {
        int p = p0, n = n0;
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < KE; ++k) {
            if (e0 + k < PN) {
                v[k] = a * src[k] + d * xr[p] * Br[n];
                part += v[k] * Cr[n];
            }
            if (++n == N || k == KE - 1) {
                if (e0 + k < PN) atomicAdd(&yrow[p], part);
                part = 0.f;
                n = 0;
                ++p;
            }
        }
    }
};

// ---------------------------------------------------------------- sequence scan
// One work-group per (sequence, head): h <- exp(dt A) h + dt x (outer) B,
// y = h C + D x over the sequence's positions, h read from and written back to
// h_io.
template <typename TIO, int KE>
__global__ __launch_bounds__(kBaseThreads) void seq_scan_kernel(
    const TIO* __restrict__ x_u, const TIO* __restrict__ dt_u, const float* __restrict__ A,
    const TIO* __restrict__ B_u, const TIO* __restrict__ C_u, const float* __restrict__ D,
    float* __restrict__ h_io, const int32_t* __restrict__ seq_len, TIO* __restrict__ y_u, int S,
    int H, int P, int N, int G) {
    extern __shared__ float s_stage[];
    RowStage rs(s_stage, P, N);
    const int seq = blockIdx.x / H, h = blockIdx.x % H;
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int len = seq_len[seq];
    if (len <= 0 || len > S) return;
    const int PN = P * N;
    float* hs = h_io + ((size_t)seq * H + h) * PN;
    StateSlice<KE> st;
    st.init(PN, N);
    st.load(hs, PN);
    const float Ah = A[h], Dh = D[h];
    for (int t0 = 0; t0 < len; t0 += kTimeChunk) {
        const int tc = min(kTimeChunk, len - t0);
        for (int i = tid; i < tc * P; i += kBaseThreads) {
            const int t = i / P, p = i - t * P;
            rs.x(t)[p] = Elem<TIO>::ld(x_u, (((size_t)seq * S + t0 + t) * H + h) * P + p);
            rs.y(t)[p] = 0.f;
        }
        for (int i = tid; i < tc * N; i += kBaseThreads) {
            const int t = i / N, n = i - t * N;
            const size_t row = (((size_t)seq * S + t0 + t) * G + g) * N + n;
            rs.B(t)[n] = Elem<TIO>::ld(B_u, row);
            rs.C(t)[n] = Elem<TIO>::ld(C_u, row);
        }
        for (int t = tid; t < tc; t += kBaseThreads)
            rs.dts[t] = Elem<TIO>::ld(dt_u, ((size_t)seq * S + t0 + t) * H + h);
        __syncthreads();
        for (int t = 0; t < tc; ++t) {
            const float d = rs.dts[t];
            st.step(st.v, __expf(d * Ah), d, rs.x(t), rs.B(t), rs.C(t), rs.y(t), PN, N);
        }
        __syncthreads();
        for (int i = tid; i < tc * P; i += kBaseThreads) {
            const int t = i / P, p = i - t * P;
            Elem<TIO>::st(y_u, (((size_t)seq * S + t0 + t) * H + h) * P + p, rs.y(t)[p] + Dh * rs.x(t)[p]);
        }
        __syncthreads();
    }
    st.store(hs, PN);
}

// ---------------------------------------------------------------- tree checks (any T <= 1024)
__device__ __forceinline__ int strided_tree_check(const int32_t* __restrict__ par, int T) {
    int bad_root = 0, bad_par = 0;
    for (int i = threadIdx.x; i < T; i += kBaseThreads) {
        const int p = gload(par + i);
        if (i == 0)
            bad_root = p != -1;
        else if (p < 0 || p >= i)
            bad_par = 1;
    }
    return (__syncthreads_or(bad_root) ? kStBadRoot : 0) | (__syncthreads_or(bad_par) ? kStBadParent : 0);
}

// ---------------------------------------------------------------- snapshots
// One work-group per (item, head): the state after every node, in node order,
// each from its parent's state (kept in registers when the parent is the node
// just processed, else read back from the snapshot this thread wrote), stored
// to states[b][h][i]; y_i = H_i C_i + D x_i.
template <typename TIO, int KE>
__global__ __launch_bounds__(kBaseThreads) void snapshot_verify_kernel(
    const TIO* __restrict__ x, const TIO* __restrict__ dt, const float* __restrict__ A,
    const TIO* __restrict__ Bm, const TIO* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ h0, const int32_t* __restrict__ parent, TIO* __restrict__ y,
    float* __restrict__ states, int32_t* __restrict__ tree_status, int T, int H, int P, int N, int G) {
    extern __shared__ float s_stage[];
    RowStage rs(s_stage, P, N);
    __shared__ int s_par[kTimeChunk];
    const int b = blockIdx.x / H, h = blockIdx.x % H;
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int32_t* par_b = parent + (size_t)b * T;
    const int st = strided_tree_check(par_b, T);
    if (h == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st) return;
    const int PN = P * N;
    float* sb = states + ((size_t)b * H + h) * T * PN;
    StateSlice<KE> cur, par;
    cur.init(PN, N);
    par.init(PN, N);
    cur.load(h0 + ((size_t)b * H + h) * PN, PN);
    const float Ah = A[h], Dh = D[h];
    for (int t0 = 0; t0 < T; t0 += kTimeChunk) {
        const int tc = min(kTimeChunk, T - t0);
        for (int i = tid; i < tc * P; i += kBaseThreads) {
            const int t = i / P, p = i - t * P;
            rs.x(t)[p] = Elem<TIO>::ld(x, (((size_t)b * T + t0 + t) * H + h) * P + p);
            rs.y(t)[p] = 0.f;
        }
        for (int i = tid; i < tc * N; i += kBaseThreads) {
            const int t = i / N, n = i - t * N;
            const size_t row = (((size_t)b * T + t0 + t) * G + g) * N + n;
            rs.B(t)[n] = Elem<TIO>::ld(Bm, row);
            rs.C(t)[n] = Elem<TIO>::ld(Cm, row);
        }
        for (int t = tid; t < tc; t += kBaseThreads) {
            rs.dts[t] = Elem<TIO>::ld(dt, ((size_t)b * T + t0 + t) * H + h);
            s_par[t] = gload(par_b + t0 + t);
        }
        __syncthreads();
        for (int t = 0; t < tc; ++t) {
            const int node = t0 + t;
            const int pn = s_par[t];
            const float d = rs.dts[t];
            if (node == 0 || pn == node - 1) {
                cur.step(cur.v, __expf(d * Ah), d, rs.x(t), rs.B(t), rs.C(t), rs.y(t), PN, N);
            } else {
                par.load(sb + (size_t)pn * PN, PN);
                cur.step(par.v, __expf(d * Ah), d, rs.x(t), rs.B(t), rs.C(t), rs.y(t), PN, N);
            }
            cur.store(sb + (size_t)node * PN, PN);
        }
        __syncthreads();
        for (int i = tid; i < tc * P; i += kBaseThreads) {
            const int t = i / P, p = i - t * P;
            Elem<TIO>::st(y, (((size_t)b * T + t0 + t) * H + h) * P + p, rs.y(t)[p] + Dh * rs.x(t)[p]);
        }
        __syncthreads();
    }
}

// One work-group per (item, head, chunk of 4096 state elements): validate the
// tree and the accepted path, then copy the last accepted node's snapshot into
// h0 (len == 0 leaves h0 unchanged; an invalid item leaves it untouched).
__global__ __launch_bounds__(kBaseThreads) void snapshot_commit_kernel(
    const float* __restrict__ states, float* __restrict__ h0, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ accepted, const int32_t* __restrict__ accepted_len, int Lmax,
    int32_t* __restrict__ tree_status, int T, int H, int PN, int chunks) {
    const int chunk = blockIdx.x % chunks;
    const int bh = blockIdx.x / chunks;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    const int32_t* par_b = parent + (size_t)b * T;
    int st = strided_tree_check(par_b, T);
    const int len = gload(accepted_len + b);
    const int32_t* acc = accepted + (size_t)b * Lmax;
    int bad = len < 0 || len > Lmax || len > T;
    if (!st && !bad) {
        for (int k = tid; k < len; k += kBaseThreads) {
            const int node = gload(acc + k);
            if (node < 0 || node >= T)
                bad = 1;
            else if (k == 0 ? node != 0 : gload(par_b + node) != gload(acc + k - 1))
                bad = 1;
        }
    }
    if (__syncthreads_or(bad)) st |= kStBadPath;
    if (h == 0 && chunk == 0 && tid == 0 && tree_status) tree_status[b] = st;
    if (st || len == 0) return;
    const int last = gload(acc + len - 1);
    const float* src = states + (((size_t)b * H + h) * T + last) * PN;
    float* dst = h0 + ((size_t)b * H + h) * PN;
    const int e1 = min(PN, (chunk + 1) * 4096);
    for (int e = chunk * 4096 + tid; e < e1; e += kBaseThreads) gstore(dst + e, gload(src + e));
}

// ---------------------------------------------------------------- launchers
hipError_t launch_unroll_plan(int batch, int T, const int32_t* parent, int Lcap, int S, int32_t* seq_nodes,
                              int32_t* seq_len, int32_t* n_leaves, int32_t* tree_status, hipStream_t stream) {
    if (T <= 256)
        unroll_plan_kernel<256><<<batch, 256, 0, stream>>>(parent, T, Lcap, S, seq_nodes, seq_len, n_leaves,
                                                           tree_status);
    else
        unroll_plan_kernel<1024><<<batch, 1024, 0, stream>>>(parent, T, Lcap, S, seq_nodes, seq_len,
                                                             n_leaves, tree_status);
    return hipGetLastError();
}

hipError_t launch_unroll_gather(const UnrollArgs& u, bool bf16, hipStream_t stream) {
    const long nseq = (long)u.batch * u.Lcap;
    const long blocks = nseq * u.S + nseq * u.H;
    if (bf16)
        unroll_gather_kernel<uint16_t><<<(unsigned)blocks, kBaseThreads, 0, stream>>>(
            (const uint16_t*)u.x, (const uint16_t*)u.dt, (const uint16_t*)u.B, (const uint16_t*)u.C, u.h0,
            u.seq_nodes, u.seq_len, u.T, u.H, u.P, u.N, u.G, u.Lcap, u.S, (int)nseq, (uint16_t*)u.x_u,
            (uint16_t*)u.dt_u, (uint16_t*)u.B_u, (uint16_t*)u.C_u, u.h0_u);
    else
        unroll_gather_kernel<float><<<(unsigned)blocks, kBaseThreads, 0, stream>>>(
            (const float*)u.x, (const float*)u.dt, (const float*)u.B, (const float*)u.C, u.h0, u.seq_nodes,
            u.seq_len, u.T, u.H, u.P, u.N, u.G, u.Lcap, u.S, (int)nseq, (float*)u.x_u, (float*)u.dt_u,
            (float*)u.B_u, (float*)u.C_u, u.h0_u);
    return hipGetLastError();
}

// elements of the state per thread: the smallest of 8, 16, 32, 64 that covers P N
template <typename TIO, template <typename, int> class K, typename... Args>
static hipError_t launch_ke(int PN, dim3 grid, hipStream_t stream, Args... args);

template <typename TIO, int KE>
static void seq_scan_launch(int nblk, hipStream_t stream, const SeqScanArgs& a) {
    seq_scan_kernel<TIO, KE><<<nblk, kBaseThreads, row_stage_bytes(a.P, a.N), stream>>>(
        (const TIO*)a.x_u, (const TIO*)a.dt_u, a.A, (const TIO*)a.B_u, (const TIO*)a.C_u, a.D, a.h_io,
        a.seq_len, (TIO*)a.y_u, a.S, a.H, a.P, a.N, a.G);
}

template <typename TIO>
static void seq_scan_dispatch(int nblk, hipStream_t stream, const SeqScanArgs& a) {
    const int PN = a.P * a.N;
    if (PN <= 8 * kBaseThreads)
        seq_scan_launch<TIO, 8>(nblk, stream, a);
    else if (PN <= 16 * kBaseThreads)
        seq_scan_launch<TIO, 16>(nblk, stream, a);
    else if (PN <= 32 * kBaseThreads)
        seq_scan_launch<TIO, 32>(nblk, stream, a);
    else
        seq_scan_launch<TIO, 64>(nblk, stream, a);
}

hipError_t launch_seq_scan(const SeqScanArgs& a, bool bf16, hipStream_t stream) {
    const int nblk = a.nseq * a.H;
    if (bf16)
        seq_scan_dispatch<uint16_t>(nblk, stream, a);
    else
        seq_scan_dispatch<float>(nblk, stream, a);
    return hipGetLastError();
}

template <typename TIO, int KE>
static void snapshot_launch(const VerifyArgs& a, float* states, hipStream_t stream) {
    snapshot_verify_kernel<TIO, KE><<<a.batch * a.H, kBaseThreads, row_stage_bytes(a.P, a.N), stream>>>(
        (const TIO*)a.x, (const TIO*)a.dt, a.A, (const TIO*)a.B, (const TIO*)a.C, a.D, a.h0, a.parent,
        (TIO*)a.y, states, a.tree_status, a.T, a.H, a.P, a.N, a.G);
}

template <typename TIO>
static void snapshot_dispatch(const VerifyArgs& a, float* states, hipStream_t stream) {
    const int PN = a.P * a.N;
    if (PN <= 8 * kBaseThreads)
        snapshot_launch<TIO, 8>(a, states, stream);
    else if (PN <= 16 * kBaseThreads)
        snapshot_launch<TIO, 16>(a, states, stream);
    else if (PN <= 32 * kBaseThreads)
        snapshot_launch<TIO, 32>(a, states, stream);
    else
        snapshot_launch<TIO, 64>(a, states, stream);
}

hipError_t launch_snapshot_verify(const VerifyArgs& a, float* states, bool bf16, hipStream_t stream) {
    if (bf16)
        snapshot_dispatch<uint16_t>(a, states, stream);
    else
        snapshot_dispatch<float>(a, states, stream);
    return hipGetLastError();
}

hipError_t launch_snapshot_commit(int batch, int T, int H, int PN, const float* states, float* h0,
                                  const int32_t* parent, const int32_t* accepted,
                                  const int32_t* accepted_len, int Lmax, int32_t* tree_status,
                                  hipStream_t stream) {
    const int chunks = (PN + 4095) / 4096;
    snapshot_commit_kernel<<<(unsigned)((long)batch * H * chunks), kBaseThreads, 0, stream>>>(
        states, h0, parent, accepted, accepted_len, Lmax, tree_status, T, H, PN, chunks);
    return hipGetLastError();
}

}  // namespace tsv
