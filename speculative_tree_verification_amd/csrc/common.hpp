// common.hpp -- device helpers shared by the tree-SSD kernels (gfx950, wave64).
//
// Tree topology of a packed draft tree ("STree: Speculative Tree Decoding for
// Hybrid State Space Models", atlas.scime.ai summary, section "Approach": the
// tree mask L over the packed sequence): node 0 is the root, every parent is
// listed before its children, T <= 1024 (the MFMA kernels take T <= 256).
// One work-group with at least one thread per node holds one tree in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsv {

constexpr int kMaxNodes = 256;       // trees the MFMA kernels take
constexpr int kMaxNodesLarge = 1024;  // trees past 256 nodes: the plain kernels

// 64-bit words of one node's ancestor bit set (node j: bit j % 64 of word j / 64)
__host__ __device__ constexpr int anc_words(int T) { return T <= 256 ? 4 : (T + 63) / 64; }
constexpr int kBlock = 256;
constexpr int kWave = 64;

constexpr int kStBadRoot = 1;
constexpr int kStBadParent = 2;
constexpr int kStBadPath = 4;
constexpr int kStBadToken = 16;  // a draft token outside the vocabulary

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (a in the low half), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Loads and stores through the global address space. A pointer read from
// memory (a caller's table) is generic to the compiler, and its generic (flat)
// accesses count against both memory counters, so every later LDS wait would
// also wait for them; these casts keep them plain global accesses.
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
    return *(const T __attribute__((address_space(1)))*)p;
}
template <typename T>
__device__ __forceinline__ void gstore(T* p, const T& v) {
    *(T __attribute__((address_space(1)))*)p = v;
}
// 16-byte vector types go through native vectors: the copy of a HIP vector
// class takes a generic reference, which would make the access flat again
typedef float gf32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t gu32x4 __attribute__((ext_vector_type(4)));
template <>
__device__ __forceinline__ float4 gload(const float4* p) {
    const gf32x4 v = *(const gf32x4 __attribute__((address_space(1)))*)p;
    return make_float4(v.x, v.y, v.z, v.w);
}
template <>
__device__ __forceinline__ uint4 gload(const uint4* p) {
    const gu32x4 v = *(const gu32x4 __attribute__((address_space(1)))*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <>
__device__ __forceinline__ void gstore(float4* p, const float4& v) {
    *(gf32x4 __attribute__((address_space(1)))*)p = gf32x4{v.x, v.y, v.z, v.w};
}
typedef uint32_t gu32x2 __attribute__((ext_vector_type(2)));
template <>
__device__ __forceinline__ uint2 gload(const uint2* p) {
    const gu32x2 v = *(const gu32x2 __attribute__((address_space(1)))*)p;
    return make_uint2(v.x, v.y);
}
template <>
__device__ __forceinline__ void gstore(uint2* p, const uint2& v) {
    *(gu32x2 __attribute__((address_space(1)))*)p = gu32x2{v.x, v.y};
}
template <>
__device__ __forceinline__ void gstore(uint4* p, const uint4& v) {
    *(gu32x4 __attribute__((address_space(1)))*)p = gu32x4{v.x, v.y, v.z, v.w};
}

// Nontemporal 16-byte global load and store, for data a launch touches once
// (a state read once and written once): it is streamed instead of being kept
// in the caches other work-groups re-read from.
__device__ __forceinline__ float4 gload_nt(const float4* p) {
    const gf32x4 v = __builtin_nontemporal_load((const gf32x4 __attribute__((address_space(1)))*)p);
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void gstore_nt(float4* p, const float4& v) {
    __builtin_nontemporal_store(gf32x4{v.x, v.y, v.z, v.w}, (gf32x4 __attribute__((address_space(1)))*)p);
}
__device__ __forceinline__ void gstore_nt(uint2* p, const uint2& v) {
    __builtin_nontemporal_store(gu32x2{v.x, v.y}, (gu32x2 __attribute__((address_space(1)))*)p);
}
__device__ __forceinline__ void gstore_nt(uint4* p, const uint4& v) {
    __builtin_nontemporal_store(gu32x4{v.x, v.y, v.z, v.w}, (gu32x4 __attribute__((address_space(1)))*)p);
}

// element access for the two input dtypes (float, or bf16 stored as uint16_t)
template <typename TIO>
struct Elem;

template <>
struct Elem<float> {
    static __device__ __forceinline__ float ld(const float* p, size_t i) { return gload(p + i); }
    static __device__ __forceinline__ void st(float* p, size_t i, float v) { gstore(p + i, v); }
};

template <>
struct Elem<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t* p, size_t i) {
        return bf16_bits_to_f32(gload(p + i));
    }
    static __device__ __forceinline__ void st(uint16_t* p, size_t i, float v) {
        gstore(p + i, f32_to_bf16_bits(v));
    }
};

// ---------------------------------------------------------------- launch helpers
// Work-groups go to the 8 XCDs (each with its own L2) in turn: block x runs on
// XCD x % 8. This renumbering gives consecutive logical indices to the blocks
// of one XCD (a bijection of [0, n)), so that neighbouring work-groups that read
// the same rows (an item's tree and B/C tile) share one L2.
__device__ __forceinline__ int xcd_block(int x, int n) {
    constexpr int kXcd = 8;
    const int q = n / kXcd, r = n % kXcd, c = x % kXcd;
    return c * q + min(c, r) + x / kXcd;
}

// ---------------------------------------------------------------- sync helpers
// Order LDS traffic between the lanes of one wave (no hardware barrier).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Work-group barrier that orders LDS traffic only: global stores still in
// flight are not waited for (a plain __syncthreads waits for every
// outstanding vector memory operation, stores included).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// OR of p over the NT threads of the block, with LDS-only barriers: global
// loads still in flight are not waited for (a __syncthreads-based reduction
// carries a work-group release fence, which on gfx9 waits for every
// outstanding vector memory operation, loads included). `s_red` holds at least
// NT/64 ints of LDS.
template <int NT>
__device__ __forceinline__ int lds_sync_or(int p, int* s_red) {
    const int wave = threadIdx.x / kWave;
    const int any = __ballot(p) != 0ull;
    if ((threadIdx.x & (kWave - 1)) == 0) s_red[wave] = any;
    lds_barrier();
    int r = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) r |= s_red[w];
    lds_barrier();  // s_red may be reused
    return r;
}

// Exclusive prefix sum over the NT threads of the block. `scratch` holds at
// least NT/64 ints of LDS. Returns the exclusive prefix; *total gets the sum.
// With LDS_ONLY the barriers order LDS traffic only (see lds_sync_or).
template <int NT = kBlock, bool LDS_ONLY = false>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) scratch[wave] = incl;
    if (LDS_ONLY)
        lds_barrier();
    else
        __syncthreads();
    int base = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        int t = scratch[w];
        if (w < wave) base += t;
        sum += t;
    }
    *total = sum;
    if (LDS_ONLY)
        lds_barrier();
    else
        __syncthreads();
    return base + incl - v;
}

// four consecutive floats of a row with `rem` >= 1 valid elements left (VEC: a
// 16-byte aligned row of a multiple of four elements)
template <bool VEC>
__device__ __forceinline__ float4 ld4(const float* __restrict__ p, int rem) {
    if (VEC) return *(const float4*)p;
    float4 r;
    r.x = p[0];
    r.y = rem > 1 ? p[1] : 0.f;
    r.z = rem > 2 ? p[2] : 0.f;
    r.w = rem > 3 ? p[3] : 0.f;
    return r;
}

// four consecutive elements of a row of q, k or v as floats (bf16 rows: VEC
// means an 8-byte aligned row of a multiple of four elements)
template <typename TIO, bool VEC>
__device__ __forceinline__ float4 ld4io(const TIO* __restrict__ p, int rem) {
    if constexpr (sizeof(TIO) == 4) {
        return ld4<VEC>((const float*)p, rem);
    } else {
        if (VEC) {
            const uint2 u = gload((const uint2*)p);
            return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
        }
        float4 r;
        r.x = Elem<TIO>::ld(p, 0);
        r.y = rem > 1 ? Elem<TIO>::ld(p, 1) : 0.f;
        r.z = rem > 2 ? Elem<TIO>::ld(p, 2) : 0.f;
        r.w = rem > 3 ? Elem<TIO>::ld(p, 3) : 0.f;
        return r;
    }
}

// ---------------------------------------------------------------- topology
// parent[threadIdx.x] of a tree (0 for threads past T; T >= 1): issue this
// load early and hand the value to check_tree, so that other loads overlap its
// latency. The load is unconditional (clamped index), which lets the compiler
// count exactly how many later loads it may leave in flight; the empty asm
// hides the pointer's provenance so that the load is not treated as invariant
// and moved next to its use, behind the loads issued after it, and the
// scheduling barrier keeps it first.
__device__ __forceinline__ int load_parent(const int32_t* parent_b, int T) {
    typedef const int32_t __attribute__((address_space(1))) gint;
    const int i = threadIdx.x;
    uint64_t u = (uint64_t)parent_b;
    asm volatile("" : "+v"(u));
    const int p = ((gint*)u)[i < T ? i : T - 1];
    __builtin_amdgcn_sched_barrier(0);
    return i < T ? p : 0;
}

// Stage the parents into LDS and validate them: returns the status bits
// (kStBadRoot | kStBadParent), identical in every thread. Acts as a barrier.
__device__ __forceinline__ int check_tree(int p, int T, int* s_par) {
    const int i = threadIdx.x;
    int bad_root = 0, bad_par = 0;
    if (i < T) {
        s_par[i] = p;
        if (i == 0)
            bad_root = (p != -1);
        else
            bad_par = (p < 0 || p >= i);
    }
    // one barrier on the common path; a second one tells the two errors apart
    if (!__syncthreads_or(bad_root | bad_par)) return 0;
    int r = __syncthreads_or(bad_root) ? kStBadRoot : 0;
    return r | (__syncthreads_or(bad_par) ? kStBadParent : 0);
}

// check_tree with LDS-only barriers: loads issued before it stay in flight.
// `s_red` holds at least NT/64 ints of LDS.
template <int NT>
__device__ __forceinline__ int check_tree_lds(int p, int T, int* s_par, int* s_red) {
    const int i = threadIdx.x;
    int bad_root = 0, bad_par = 0;
    if (i < T) {
        s_par[i] = p;
        if (i == 0)
            bad_root = (p != -1);
        else
            bad_par = (p < 0 || p >= i);
    }
    // one reduction on the common path; a second one tells the two errors apart
    if (!lds_sync_or<NT>(bad_root | bad_par, s_red)) return 0;
    int r = lds_sync_or<NT>(bad_root, s_red) ? kStBadRoot : 0;
    return r | (lds_sync_or<NT>(bad_par, s_red) ? kStBadParent : 0);
}

// load_parent + check_tree in one step.
__device__ __forceinline__ int load_tree(const int32_t* __restrict__ parent_b, int T,
                                         int* s_par) {
    return check_tree(load_parent(parent_b, T), T, s_par);
}

// Depth of node threadIdx.x for shallow trees: each thread walks to the root
// through the parents in LDS (no barrier per step), at most kWalkDepth steps;
// if some node is deeper, pointer jumping takes over. All barriers are
// LDS-only, so global loads issued earlier stay in flight. s_nxt, s_dep: LDS
// scratch of at least T ints; s_red: NT/64 ints.
constexpr int kWalkDepth = 16;
template <int NT>
__device__ __forceinline__ int tree_depth_shallow(const int* s_par, int T, int* s_nxt, int* s_dep,
                                                  int* s_red) {
    const int i = threadIdx.x;
    int d = 0, j = i < T ? s_par[i] : -1;
#pragma unroll 1
    for (int k = 0; k < kWalkDepth && j >= 0; ++k) {
        ++d;
        j = s_par[j];
    }
    if (!lds_sync_or<NT>(j >= 0, s_red)) return i < T ? d : 0;
    // pointer jumping: after round r every node knows its distance to the
    // ancestor 2^r steps up
    int nxt = -1, dep = 0;
    if (i < T) {
        nxt = s_par[i];
        dep = (nxt >= 0) ? 1 : 0;
        s_nxt[i] = nxt;
        s_dep[i] = dep;
    }
    while (lds_sync_or<NT>(nxt >= 0, s_red)) {
        int n2 = nxt, d2 = dep;
        if (nxt >= 0) {
            d2 = dep + s_dep[nxt];
            n2 = s_nxt[nxt];
        }
        lds_barrier();
        if (i < T) {
            s_dep[i] = d2;
            s_nxt[i] = n2;
        }
        nxt = n2;
        dep = d2;
    }
    return dep;
}

// Depth (edges from the root) of node threadIdx.x by pointer jumping over the
// validated tree in LDS: after round r every node knows its distance to the
// ancestor 2^r steps up. At most ceil(log2 T) rounds; stops early when every
// node has reached the root. s_nxt and s_dep are LDS scratch of kMaxNodes.
__device__ __forceinline__ int tree_depth(const int* s_par, int T, int* s_nxt, int* s_dep) {
    const int i = threadIdx.x;
    int nxt = -1, dep = 0;
    if (i < T) {
        nxt = s_par[i];
        dep = (nxt >= 0) ? 1 : 0;
        s_nxt[i] = nxt;
        s_dep[i] = dep;
    }
    while (__syncthreads_or(nxt >= 0)) {
        int n2 = nxt, d2 = dep;
        if (nxt >= 0) {
            d2 = dep + s_dep[nxt];
            n2 = s_nxt[nxt];
        }
        __syncthreads();
        if (i < T) {
            s_dep[i] = d2;
            s_nxt[i] = n2;
        }
        nxt = n2;
        dep = d2;
    }
    return dep;
}

}  // namespace tsv
