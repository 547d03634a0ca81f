/*
 * HSTU attention oracle: a plain, slow fp64 CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code with the HIP kernels.
 *
 * What it computes is the definition on the HSTU Attention page ("Overview",
 * the four displayed equations), per packed sequence b and head h:
 *
 *     S = alpha * Q K^T,   A = (M (.) SiLU(S)) / L_scale,   O = A V,
 *
 * with no softmax and no row normalisation ("Overview", the paragraph after the
 * equations).  Packed THD layout and cumulative offsets follow the page's
 * "Tensor layout" table.  The mask M is the page's "Mask support" table: a
 * token window (left, right) in which -1 leaves a side unbounded, so (-1,-1) is
 * full attention, (-1,0) causal, and finite bounds give a local (sliding)
 * window; or the table's arbitrary mask: per packed query row r, endpoints
 * F0, F1, ..., F_{N-1} (N odd) read from func[n * ld + r] make the visible keys
 * [0, F0) u [F1, F2) u [F3, F4) u ..., each interval taken on its own (they may
 * overlap or come in any order, and an interval whose end is not above its
 * start is empty); keys outside the sequence stay invisible.
 *
 * Readings where the page is silent (each is listed in the design notes):
 *  - window_size follows the FlashAttention-2 convention, the one the cuDNN
 *    SDPA page maps its own diagonal band bounds onto (PyTorch custom ops,
 *    the band conventions): key j is visible to query i iff
 *    i - left <= j <= i + right, a negative bound dropping its side.  In the
 *    SDPA page's terms our left is its left bound minus one and our right is
 *    its right bound; (-1, 0) is then exactly causal, as the HSTU page says;
 *  - the band is top-left aligned inside each sequence: i and j are local
 *    indices counted from the sequence's first query and first key, so causal
 *    (-1, 0) means j <= i.  All measured workloads have equal query and key
 *    lengths, where top-left and bottom-right agree;
 *  - the arbitrary mask's endpoints are local key indices like j (the union
 *    starts at key 0 of the sequence), indexed by the packed (global) query row;
 *  - L_scale is one global scalar for the whole call (the page calls it a
 *    runtime normalisation factor, not a per-sequence token count);
 *  - a query row with no visible key gets O = 0, a key row seen by no query
 *    gets dK = dV = 0 (the page's zero-write rule for empty tiles).
 *
 * The backward is the chain rule applied to that definition, with dO the
 * upstream gradient of O:
 *
 *     dV[j]  = sum_i M_ij SiLU(s_ij)/L * dO[i]
 *     dA_ij  = dO[i] . V[j]
 *     dS_ij  = dA_ij * SiLU'(s_ij) / L,   SiLU'(s) = sig(s) (1 + s (1 - sig(s)))
 *     dQ[i]  = sum_j M_ij alpha dS_ij K[j]
 *     dK[j]  = sum_i M_ij alpha dS_ij Q[i]
 *
 * Every output row is computed on its own, straight from those sums, in fp64
 * with libm exp; rows are independent so they are spread over OpenMP threads,
 * which does not change any sum's order.  Built with -O2 and no fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Index of element (token t, head h, dim d) of a packed (T, H, D) tensor. */
static inline size_t thd(int64_t t, int64_t h, int64_t d, int64_t H, int64_t D) {
    return ((size_t)t * (size_t)H + (size_t)h) * (size_t)D + (size_t)d;
}

/* Sequence that owns packed row r: the b with cu[b] <= r < cu[b+1]. */
static int64_t owner(const int32_t* cu, int64_t B, int64_t r) {
    for (int64_t b = 0; b < B; ++b)
        if (cu[b] <= r && r < cu[b + 1]) return b;
    return -1;
}

/* The mask: a token window (left, right), a negative bound meaning that side
 * is unbounded, or, when func is not NULL, the interval list of each query row
 * (func_n endpoints, row r's n-th at func[n * func_ld + r]). */
typedef struct {
    int64_t left, right;
    const int32_t* func;
    int64_t func_n, func_ld;
} mask_t;

/* M_ij for packed query row r = local query index i of its sequence, and local
 * key index j (0 <= j < L_k). */
static inline int visible(const mask_t* m, int64_t r, int64_t i, int64_t j) {
    if (m->func) {
        const int32_t* f = m->func + r;
        if (j < f[0]) return 1;
        for (int64_t n = 1; n + 1 < m->func_n; n += 2)
            if (f[n * m->func_ld] <= j && j < f[(n + 1) * m->func_ld]) return 1;
        return 0;
    }
    if (m->left >= 0 && j < i - m->left) return 0;
    if (m->right >= 0 && j > i + m->right) return 0;
    return 1;
}

static inline double dot(const double* x, const double* y, int64_t D) {
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += x[d] * y[d];
    return acc;
}

static inline double sigmoid(double s) { return 1.0 / (1.0 + exp(-s)); }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Forward: out[n, h, :] = O[rows[n], h, :] for n < nrows.
 * rows == NULL means all T_q rows in order (nrows must then equal T_q).
 * Returns 0, or -1 if a row is outside every sequence.
 */
int oracle_hstu_fwd(int64_t B, const int32_t* cu_q, const int32_t* cu_k, int64_t H, int64_t D,
                    const double* q, const double* k, const double* v,
                    double alpha, double ls, int64_t left, int64_t right,
                    const int32_t* func, int64_t func_n, int64_t func_ld,
                    const int64_t* rows, int64_t nrows, double* out) {
    const mask_t mk = {left, right, func, func_n, func_ld};
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2) reduction(| : bad)
    for (int64_t n = 0; n < nrows; ++n) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t r = rows ? rows[n] : n;
            double* o = out + thd(n, h, 0, H, D);
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            const int64_t b = owner(cu_q, B, r);
            if (b < 0) { bad = 1; continue; }
            const int64_t i = r - cu_q[b];
            const int64_t k0 = cu_k[b], lk = (int64_t)cu_k[b + 1] - cu_k[b];
            const double* qi = q + thd(r, h, 0, H, D);
            for (int64_t j = 0; j < lk; ++j) {
                if (!visible(&mk, r, i, j)) continue;
                const double s = alpha * dot(qi, k + thd(k0 + j, h, 0, H, D), D);
                const double a = s * sigmoid(s) / ls;
                const double* vj = v + thd(k0 + j, h, 0, H, D);
                for (int64_t d = 0; d < D; ++d) o[d] += a * vj[d];
            }
        }
    }
    return bad ? -1 : 0;
}

/* dQ rows: dq[n, h, :] = dQ[rows[n], h, :]. */
int oracle_hstu_bwd_dq(int64_t B, const int32_t* cu_q, const int32_t* cu_k, int64_t H, int64_t D,
                       const double* dout, const double* q, const double* k, const double* v,
                       double alpha, double ls, int64_t left, int64_t right,
                    const int32_t* func, int64_t func_n, int64_t func_ld,
                       const int64_t* rows, int64_t nrows, double* dq) {
    const mask_t mk = {left, right, func, func_n, func_ld};
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2) reduction(| : bad)
    for (int64_t n = 0; n < nrows; ++n) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t r = rows ? rows[n] : n;
            double* g = dq + thd(n, h, 0, H, D);
            for (int64_t d = 0; d < D; ++d) g[d] = 0.0;
            const int64_t b = owner(cu_q, B, r);
            if (b < 0) { bad = 1; continue; }
            const int64_t i = r - cu_q[b];
            const int64_t k0 = cu_k[b], lk = (int64_t)cu_k[b + 1] - cu_k[b];
            const double* qi = q + thd(r, h, 0, H, D);
            const double* doi = dout + thd(r, h, 0, H, D);
            for (int64_t j = 0; j < lk; ++j) {
                if (!visible(&mk, r, i, j)) continue;
                const double* kj = k + thd(k0 + j, h, 0, H, D);
                const double s = alpha * dot(qi, kj, D);
                const double sg = sigmoid(s);
                const double da = dot(doi, v + thd(k0 + j, h, 0, H, D), D);
                const double ds = da * sg * (1.0 + s * (1.0 - sg)) / ls;
                for (int64_t d = 0; d < D; ++d) g[d] += alpha * ds * kj[d];
            }
        }
    }
    return bad ? -1 : 0;
}

/* dK and dV rows: dk/dv[n, h, :] = dK/dV[rows[n], h, :] for packed key rows. */
int oracle_hstu_bwd_dkdv(int64_t B, const int32_t* cu_q, const int32_t* cu_k, int64_t H, int64_t D,
                         const double* dout, const double* q, const double* k, const double* v,
                         double alpha, double ls, int64_t left, int64_t right,
                    const int32_t* func, int64_t func_n, int64_t func_ld,
                         const int64_t* rows, int64_t nrows, double* dk, double* dv) {
    const mask_t mk = {left, right, func, func_n, func_ld};
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2) reduction(| : bad)
    for (int64_t n = 0; n < nrows; ++n) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t r = rows ? rows[n] : n;
            double* gk = dk + thd(n, h, 0, H, D);
            double* gv = dv + thd(n, h, 0, H, D);
            for (int64_t d = 0; d < D; ++d) { gk[d] = 0.0; gv[d] = 0.0; }
            const int64_t b = owner(cu_k, B, r);
            if (b < 0) { bad = 1; continue; }
            const int64_t j = r - cu_k[b];
            const int64_t q0 = cu_q[b], lq = (int64_t)cu_q[b + 1] - cu_q[b];
            const double* kj = k + thd(r, h, 0, H, D);
            const double* vj = v + thd(r, h, 0, H, D);
            for (int64_t i = 0; i < lq; ++i) {
                if (!visible(&mk, q0 + i, i, j)) continue;
                const double* qi = q + thd(q0 + i, h, 0, H, D);
                const double* doi = dout + thd(q0 + i, h, 0, H, D);
                const double s = alpha * dot(qi, kj, D);
                const double sg = sigmoid(s);
                const double a = s * sg / ls;
                const double da = dot(doi, vj, D);
                const double ds = da * sg * (1.0 + s * (1.0 - sg)) / ls;
                for (int64_t d = 0; d < D; ++d) {
                    gv[d] += a * doi[d];
                    gk[d] += alpha * ds * qi[d];
                }
            }
        }
    }
    return bad ? -1 : 0;
}
