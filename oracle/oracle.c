/*
 * oracle.c -- plain fp64 CPU oracle for packed-tree SSD (Mamba2) verification
 * and commit.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (method: "STree: Speculative Tree Decoding for Hybrid State
 * Space Models", atlas.scime.ai summary, sections "Problem" and "Approach";
 * mlsanity abstract):
 *   A draft token tree is packed into one sequence of T nodes (node 0 = root,
 *   parents before children). Every node's output must equal what the ordinary
 *   SSM recurrence gives when the root-to-node path is run as a sequence on its
 *   own: the packed pass must be exact, not an approximation of the unrolled
 *   paths. The recurrence of one Mamba2/SSD head
 *   with scalar decay A, step dt, input x (P), in/out projections B, C (N) and
 *   state H (P x N) is
 *       H <- exp(dt*A) * H + dt * x (outer) B,      y = H . C + D * x.
 *   The state before the root is the shared initial state h0.
 *   Commit rebuilds the state at the end of the accepted root path by running
 *   the same recurrence along it again (the summary restores state by
 *   replaying the accepted tokens' activations, keeping no per-node state).
 *
 * oracle_verify / oracle_commit do exactly that, literally: they unroll every
 * root-to-node path and run the sequential recurrence in double precision.
 * oracle_packed_verify is a second, independent formulation used only to check
 * the first: the packed-tree closed form with an explicit ancestor mask L and
 * accumulated log-decays cum = L * (dt*A) (the summary's formula A_tree = L log A,
 * read as the log of the per-token discrete transition exp(dt*A)).
 *
 * Every problem instance ("slice") is one (batch item, head): its own tree,
 * inputs x [T][P], dt [T], scalar A and D, B and C [T][N] (the head's group),
 * h0 [P][N]. Layouts are row-major. Status bits per slice:
 *   1 = bad root (parent[0] != -1), 2 = a parent out of range or not earlier
 *   than its child, 4 = bad accepted path. A slice with any bit set is left
 *   untouched in the outputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BAD_ROOT 1
#define ORC_BAD_PARENT 2
#define ORC_BAD_PATH 4

/* Tree check: node 0 is the root, every other node's parent is an earlier
 * node (the packed sequence lists parents before children). */
int oracle_tree_check(int T, const int32_t* parent) {
    int st = 0;
    if (T <= 0) return 0;
    if (parent[0] != -1) st |= ORC_BAD_ROOT;
    for (int i = 1; i < T; ++i)
        if (parent[i] < 0 || parent[i] >= i) st |= ORC_BAD_PARENT;
    return st;
}

/* Root path of node i, root first; returns its length (depth + 1). */
static int path_to(const int32_t* parent, int i, int* path) {
    int len = 0;
    for (int j = i; j >= 0; j = parent[j]) path[len++] = j;
    for (int a = 0, b = len - 1; a < b; ++a, --b) {
        int t = path[a]; path[a] = path[b]; path[b] = t;
    }
    return len;
}

/* Depth (edges from the root) and ancestor-or-self bit set of every node, by
 * walking each node's parent chain. Node j is bit j % 64 of word j / 64 of a
 * row of W words (W >= ceil(T / 64); the library uses max(4, ceil(T / 64))). */
void oracle_tree_info(int n_items, int T, int W, const int32_t* parent, int32_t* depth,
                      uint64_t* anc, int32_t* status) {
    for (int s = 0; s < n_items; ++s) {
        const int32_t* par = parent + (size_t)s * T;
        int st = oracle_tree_check(T, par);
        status[s] = st;
        if (st) continue;
        for (int i = 0; i < T; ++i) {
            uint64_t* a = anc + ((size_t)s * T + i) * W;
            for (int w = 0; w < W; ++w) a[w] = 0;
            int d = -1;
            for (int j = i; j >= 0; j = par[j]) {
                a[j >> 6] |= (uint64_t)1 << (j & 63);
                ++d;
            }
            depth[(size_t)s * T + i] = d;
        }
    }
}

/* One recurrence step on the P x N state S with token k of a slice. */
static void step(double* S, int P, int N, double dtk, double A, const double* xk,
                 const double* Bk) {
    double decay = exp(dtk * A);
    for (int p = 0; p < P; ++p)
        for (int n = 0; n < N; ++n)
            S[p * N + n] = decay * S[p * N + n] + dtk * xk[p] * Bk[n];
}

/* Unrolled verification: for every slice and node, run the recurrence along
 * the node's root path from h0 and read out y = S . C_i + D * x_i. */
void oracle_verify(int n, int T, int P, int N, const double* x, const double* dt,
                   const double* A, const double* Bm, const double* Cm, const double* D,
                   const double* h0, const int32_t* parent, double* y, int32_t* status) {
    for (int s = 0; s < n; ++s) status[s] = oracle_tree_check(T, parent + (size_t)s * T);
    long total = (long)n * T;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)P * N);
        int* path = (int*)malloc(sizeof(int) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(dynamic, 1)
        for (long job = 0; job < total; ++job) {
            int s = (int)(job / T), i = (int)(job % T);
            if (status[s]) continue;
            const int32_t* par = parent + (size_t)s * T;
            const double* xs = x + (size_t)s * T * P;
            const double* dts = dt + (size_t)s * T;
            const double* Bs = Bm + (size_t)s * T * N;
            const double* Cs = Cm + (size_t)s * T * N;
            memcpy(S, h0 + (size_t)s * P * N, sizeof(double) * (size_t)P * N);
            int len = path_to(par, i, path);
            for (int k = 0; k < len; ++k) {
                int j = path[k];
                step(S, P, N, dts[j], A[s], xs + (size_t)j * P, Bs + (size_t)j * N);
            }
            double* yi = y + ((size_t)s * T + i) * P;
            for (int p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int c = 0; c < N; ++c) acc += S[p * N + c] * Cs[(size_t)i * N + c];
                yi[p] = acc + D[s] * xs[(size_t)i * P + p];
            }
        }
        free(S);
        free(path);
    }
}

/* Accepted-path check: the list starts at the root and each entry is the
 * child of the previous one; 0 <= len <= Lmax. */
static int path_check(int T, const int32_t* par, const int32_t* acc, int len, int Lmax) {
    if (len < 0 || len > Lmax) return ORC_BAD_PATH;
    if (len == 0) return 0;
    if (acc[0] != 0) return ORC_BAD_PATH;
    for (int k = 1; k < len; ++k) {
        if (acc[k] < 0 || acc[k] >= T) return ORC_BAD_PATH;
        if (par[acc[k]] != acc[k - 1]) return ORC_BAD_PATH;
    }
    return 0;
}

/* Commit (activation replay): run the recurrence along the accepted path from
 * h0 and return the final state; an empty path leaves h0 unchanged. */
void oracle_commit(int n, int T, int P, int N, const double* x, const double* dt,
                   const double* A, const double* Bm, const double* h0,
                   const int32_t* parent, const int32_t* accepted, const int32_t* accepted_len,
                   int Lmax, double* h_out, int32_t* status) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < n; ++s) {
        const int32_t* par = parent + (size_t)s * T;
        const int32_t* acc = accepted + (size_t)s * Lmax;
        int st = oracle_tree_check(T, par);
        if (!st) st |= path_check(T, par, acc, accepted_len[s], Lmax);
        status[s] = st;
        if (st) continue;
        double* S = h_out + (size_t)s * P * N;
        memcpy(S, h0 + (size_t)s * P * N, sizeof(double) * (size_t)P * N);
        for (int k = 0; k < accepted_len[s]; ++k) {
            int j = acc[k];
            step(S, P, N, dt[(size_t)s * T + j], A[s], x + ((size_t)s * T + j) * P,
                 Bm + ((size_t)s * T + j) * N);
        }
    }
}

/* Packed-tree closed form (second formulation, for checking the first):
 *   L[i][j]  = 1 iff j is on the root path of i (ancestor or self)
 *   cum      = L * a,  a_j = dt_j * A
 *   Y        = ((C B^T) o exp(cum_i - cum_j) o L) diag(dt) X
 *              + diag(exp(cum)) C h0^T + D X
 * Built with explicit T x T matrices; exp is evaluated on ancestor pairs only. */
void oracle_packed_verify(int n, int T, int P, int N, const double* x, const double* dt,
                          const double* A, const double* Bm, const double* Cm,
                          const double* D, const double* h0, const int32_t* parent,
                          double* y, int32_t* status) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < n; ++s) {
        const int32_t* par = parent + (size_t)s * T;
        int st = oracle_tree_check(T, par);
        status[s] = st;
        if (st || T == 0) continue;
        const double* xs = x + (size_t)s * T * P;
        const double* dts = dt + (size_t)s * T;
        const double* Bs = Bm + (size_t)s * T * N;
        const double* Cs = Cm + (size_t)s * T * N;
        const double* H0 = h0 + (size_t)s * P * N;
        unsigned char* L = (unsigned char*)calloc((size_t)T * T, 1);
        double* cum = (double*)calloc((size_t)T, sizeof(double));
        double* M = (double*)calloc((size_t)T * T, sizeof(double));
        for (int i = 0; i < T; ++i)
            for (int j = i; j >= 0; j = par[j]) L[(size_t)i * T + j] = 1;
        for (int i = 0; i < T; ++i) {
            double c = 0.0;
            for (int j = 0; j < T; ++j)
                if (L[(size_t)i * T + j]) c += dts[j] * A[s];
            cum[i] = c;
        }
        for (int i = 0; i < T; ++i)
            for (int j = 0; j < T; ++j) {
                if (!L[(size_t)i * T + j]) continue;
                double g = 0.0;
                for (int c = 0; c < N; ++c) g += Cs[(size_t)i * N + c] * Bs[(size_t)j * N + c];
                M[(size_t)i * T + j] = g * exp(cum[i] - cum[j]) * dts[j];
            }
        for (int i = 0; i < T; ++i) {
            double e = exp(cum[i]);
            for (int p = 0; p < P; ++p) {
                double intra = 0.0;
                for (int j = 0; j < T; ++j) intra += M[(size_t)i * T + j] * xs[(size_t)j * P + p];
                double ch = 0.0;
                for (int c = 0; c < N; ++c) ch += Cs[(size_t)i * N + c] * H0[(size_t)p * N + c];
                y[((size_t)s * T + i) * P + p] = intra + e * ch + D[s] * xs[(size_t)i * P + p];
            }
        }
        free(L);
        free(cum);
        free(M);
    }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int t) {
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}
