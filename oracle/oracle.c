/*
 * oracle.c -- plain, slow, fp64 CPU oracle for SATA causal self-attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or constant with the HIP library.
 *
 * Method: Heinsen & Kozachkov, "Self-Attention at Constant Cost per Token via
 * Symmetry-Aware Taylor Approximation" (arXiv:2602.00294), as described on the
 * blog.hotdry.top post "self-attention-constant-cost-taylor-approximation"
 * (2026-02-05), cited below as [TA] with its section headings:
 *   [TA Taylor]   "The mathematical breakthrough of the Taylor approximation"
 *   [TA Features] "Feature maps and linear attention"
 *   [TA Size]     "Hidden-state size and compute analysis"
 *   [TA Precision]"Trading precision for efficiency"
 * and the companion post "constant-cost-attention-hardware-optimization" [HW],
 * section "Rebalancing compute density and memory bandwidth" [HW Compute].
 *
 * Everything is written from the definitions, in fp64, with plain loops:
 *   - tables by brute force over all d^p ordered index tuples;
 *   - features as the literal product over a table row (no prefix reuse);
 *   - y by the O(n^2) direct form of the truncated Taylor kernel;
 *   - the state as the literal sum of outer products phi(k_t) [v_t | 1]^T;
 *   - exact softmax attention, for the truncation-error report only.
 * OpenMP parallelises only over independent outputs (heads, rows, features).
 *
 * Array layouts (all row-major, contiguous):
 *   q, k : [heads][n][dK]     v : [heads][n][dV]     y : [heads][n][dV]
 *   state: [dV+1][M] for one head, column j = dV is the normaliser Z.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Tables [TA Taylor], [TA Features]                                          */
/* ------------------------------------------------------------------------- */

/*
 * Unique monomials of the p-th tensor power of a d-vector.  [TA Taylor] keeps
 * only the index tuples of the "upper triangle" i1 <= i2 <= ... <= ip (the d=2,
 * p=2 example merges q1 q2 k1 k2 with q2 q1 k2 k1); [TA Features] defines C_p as
 * how many times each unique monomial occurs in the full expansion.
 *
 * Brute force, straight from those two sentences: walk all d^p ordered tuples,
 * sort each one ascending, and count how often each sorted tuple occurs.  A
 * sorted tuple is keyed by its base-d value, so increasing keys are exactly the
 * lexicographic order of the sorted tuples (the row order fixed for M_p).
 *
 * Returns m_p, the number of unique tuples, or -1 if d^p is too large to
 * enumerate.  If M_out is non-NULL it receives m_p rows of p int32 indices
 * (0-based); if C_out is non-NULL it receives the m_p counts.  p = 0 gives a
 * single empty tuple with count 1.
 */
int64_t oracle_tables(int d, int p, int32_t *M_out, int64_t *C_out)
{
    if (d < 1 || p < 0) return -1;
    int64_t total = 1;
    for (int r = 0; r < p; ++r) {
        total *= d;
        if (total > ((int64_t)1 << 28)) return -1;
    }
    int64_t *count = (int64_t *)calloc((size_t)total, sizeof(int64_t));
    if (!count) return -1;

    int tuple[16], sorted[16];
    memset(tuple, 0, sizeof tuple);
    for (int64_t it = 0; it < total; ++it) {
        /* current ordered tuple = digits of it in base d */
        int64_t rest = it;
        for (int r = p - 1; r >= 0; --r) { tuple[r] = (int)(rest % d); rest /= d; }
        for (int r = 0; r < p; ++r) sorted[r] = tuple[r];
        for (int a = 1; a < p; ++a)            /* insertion sort, p is tiny */
            for (int b = a; b > 0 && sorted[b - 1] > sorted[b]; --b) {
                int s = sorted[b]; sorted[b] = sorted[b - 1]; sorted[b - 1] = s;
            }
        int64_t key = 0;
        for (int r = 0; r < p; ++r) key = key * d + sorted[r];
        count[key] += 1;
    }

    int64_t m = 0;
    for (int64_t key = 0; key < total; ++key) {
        if (count[key] == 0) continue;
        if (M_out) {
            int64_t rest = key;
            for (int r = p - 1; r >= 0; --r) {
                M_out[m * p + r] = (int32_t)(rest % d);
                rest /= d;
            }
        }
        if (C_out) C_out[m] = count[key];
        ++m;
    }
    free(count);
    return m;
}

/*
 * phi_p(x)[r] = product of x[i] over the p indices i in row r of M_p
 * ([TA Features]; [HW Compute] writes it as x[..., M].prod(dim=-1)).
 * The empty product (p = 0) is 1.
 */
void oracle_features(int p, const int32_t *M, int64_t m, const double *x, double *out)
{
    for (int64_t r = 0; r < m; ++r) {
        double prod = 1.0;
        for (int s = 0; s < p; ++s) prod *= x[M[r * p + s]];
        out[r] = prod;
    }
}

/* alpha_p = 1 / (p! c^p) with c = sqrt(dK)  [TA Taylor], [TA Precision]. */
static double alpha(int p, int dK)
{
    double fact = 1.0;
    for (int s = 2; s <= p; ++s) fact *= s;
    return 1.0 / (fact * pow(sqrt((double)dK), p));
}

double oracle_alpha(int p, int dK) { return alpha(p, dK); }

/* ------------------------------------------------------------------------- */
/* Direct form                                                                */
/* ------------------------------------------------------------------------- */

/*
 * Truncated kernel w(q,k) = sum_{p=0}^{P-1} alpha_p (q.k)^p  [TA Features], and
 * causal attention with it: y_T = sum_{t<=T} w(q_T,k_t) v_t / sum_{t<=T} w(q_T,k_t).
 * The sum includes t = T (the recurrence of [TA Features] runs t = 1..T).
 * den_out (nullable) receives the denominator of every row.
 */
/* One output row of the direct form: y_T = sum_{t<=T} w(q_T,k_t) v_t / sum_{t<=T} w(q_T,k_t)
 * for one head (q, k, v point at that head's rows). */
static double direct_row(const double *q, const double *k, const double *v, int64_t T,
                         int dK, int dV, int P, const double *a, double *yT)
{
    const double *qT = q + T * dK;
    double den = 0.0;
    for (int j = 0; j < dV; ++j) yT[j] = 0.0;
    for (int64_t t = 0; t <= T; ++t) {
        const double *kt = k + t * dK;
        const double *vt = v + t * dV;
        double x = 0.0;
        for (int i = 0; i < dK; ++i) x += qT[i] * kt[i];
        double w = 0.0, xp = 1.0;
        for (int p = 0; p < P; ++p) { w += a[p] * xp; xp *= x; }
        den += w;
        for (int j = 0; j < dV; ++j) yT[j] += w * vt[j];
    }
    for (int j = 0; j < dV; ++j) yT[j] /= den;
    return den;
}

void oracle_direct(const double *q, const double *k, const double *v,
                   int64_t heads, int64_t n, int dK, int dV, int P,
                   double *y, double *den_out)
{
    double a[32];
    for (int p = 0; p < P && p < 32; ++p) a[p] = alpha(p, dK);

#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t h = 0; h < heads; ++h) {
        for (int64_t T = 0; T < n; ++T) {
            const double den = direct_row(q + h * n * dK, k + h * n * dK, v + h * n * dV, T,
                                          dK, dV, P, a, y + (h * n + T) * dV);
            if (den_out) den_out[h * n + T] = den;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Gradients of the direct form                                               */
/* ------------------------------------------------------------------------- */

/*
 * For a loss L = sum_T dy_T . y_T with y the direct form above, the chain rule through
 * y_T = N_T / D_T (N_T = sum_{t<=T} w_Tt v_t, D_T = sum_{t<=T} w_Tt, w_Tt = w(q_T.k_t))
 * gives dL/dN_T = g_T = dy_T / D_T and dL/dD_T = h_T = -(dy_T . y_T) / D_T, so that
 * dL/dw_Tt = c_Tt = g_T . v_t + h_T and
 *   dv_t = sum_{T>=t} w_Tt g_T,
 *   dq_T = sum_{t<=T} c_Tt w'(x_Tt) k_t,      dk_t = sum_{T>=t} c_Tt w'(x_Tt) q_T,
 * with x_Tt = q_T.k_t and w'(x) = sum_{p=1}^{P-1} p alpha_p x^{p-1}.  Written out pair by
 * pair, O(n^2) per head; heads in parallel.  q, k, dq, dk: [heads][n][dK]; v, dy, dv:
 * [heads][n][dV].
 */
void oracle_direct_grad(const double *q, const double *k, const double *v, const double *dy,
                        int64_t heads, int64_t n, int dK, int dV, int P,
                        double *dq, double *dk, double *dv)
{
    double a[32];
    for (int p = 0; p < P && p < 32; ++p) a[p] = alpha(p, dK);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < heads; ++h) {
        const double *qh = q + h * n * dK, *kh = k + h * n * dK;
        const double *vh = v + h * n * dV, *dyh = dy + h * n * dV;
        double *dqh = dq + h * n * dK, *dkh = dk + h * n * dK, *dvh = dv + h * n * dV;
        double *yT = (double *)malloc((size_t)dV * sizeof(double));
        double *gT = (double *)malloc((size_t)dV * sizeof(double));
        for (int64_t i = 0; i < n * dK; ++i) { dqh[i] = 0.0; dkh[i] = 0.0; }
        for (int64_t i = 0; i < n * dV; ++i) dvh[i] = 0.0;
        for (int64_t T = 0; T < n; ++T) {
            const double den = direct_row(qh, kh, vh, T, dK, dV, P, a, yT);
            const double *dyT = dyh + T * dV;
            double hT = 0.0;
            for (int j = 0; j < dV; ++j) {
                gT[j] = dyT[j] / den;
                hT -= dyT[j] * yT[j];
            }
            hT /= den;
            const double *qT = qh + T * dK;
            for (int64_t t = 0; t <= T; ++t) {
                const double *kt = kh + t * dK;
                const double *vt = vh + t * dV;
                double x = 0.0;
                for (int i = 0; i < dK; ++i) x += qT[i] * kt[i];
                double w = 0.0, wp = 0.0, xp = 1.0;
                for (int p = 0; p < P; ++p) {
                    w += a[p] * xp;
                    if (p + 1 < P) wp += (p + 1) * a[p + 1] * xp;
                    xp *= x;
                }
                double c = hT;
                for (int j = 0; j < dV; ++j) c += gT[j] * vt[j];
                for (int j = 0; j < dV; ++j) dvh[t * dV + j] += w * gT[j];
                for (int i = 0; i < dK; ++i) {
                    dqh[T * dK + i] += c * wp * kt[i];
                    dkh[t * dK + i] += c * wp * qT[i];
                }
            }
        }
        free(yT);
        free(gT);
    }
}

/* Sampled rows of the direct form: out[r] = y of token rows[r] of head heads_of[r]
 * (q, k: [heads][n][dK], v: [heads][n][dV]); each row costs O(T (dK + dV)). */
void oracle_direct_rows(const double *q, const double *k, const double *v,
                        int64_t n, int dK, int dV, int P,
                        const int64_t *heads_of, const int64_t *rows, int64_t nr, double *out)
{
    double a[32];
    for (int p = 0; p < P && p < 32; ++p) a[p] = alpha(p, dK);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nr; ++r) {
        const int64_t h = heads_of[r];
        direct_row(q + h * n * dK, k + h * n * dK, v + h * n * dV, rows[r], dK, dV, P, a,
                   out + r * dV);
    }
}

/* ------------------------------------------------------------------------- */
/* Feature form: the fixed-size state and its readout                         */
/* ------------------------------------------------------------------------- */

/* Concatenated tables for p = 0..P-1: feature f has degree deg[f], indices
 * idx[f*P .. f*P+deg-1] and multiplicity cnt[f].  Built from oracle_tables. */
typedef struct {
    int64_t M;
    int P;
    int *deg;
    int32_t *idx;
    int64_t *cnt;
} feat_list;

static int feat_list_build(int dK, int P, feat_list *fl)
{
    int64_t M = 0, mp[32];
    for (int p = 0; p < P; ++p) {
        mp[p] = oracle_tables(dK, p, NULL, NULL);
        if (mp[p] < 0) return -1;
        M += mp[p];
    }
    fl->M = M;
    fl->P = P;
    fl->deg = (int *)malloc(sizeof(int) * (size_t)M);
    fl->idx = (int32_t *)calloc((size_t)(M * (P > 0 ? P : 1)), sizeof(int32_t));
    fl->cnt = (int64_t *)malloc(sizeof(int64_t) * (size_t)M);
    if (!fl->deg || !fl->idx || !fl->cnt) return -1;
    int64_t f0 = 0;
    for (int p = 0; p < P; ++p) {
        int32_t *Mp = (int32_t *)malloc(sizeof(int32_t) * (size_t)(mp[p] * (p > 0 ? p : 1)));
        oracle_tables(dK, p, Mp, fl->cnt + f0);
        for (int64_t r = 0; r < mp[p]; ++r) {
            fl->deg[f0 + r] = p;
            for (int s = 0; s < p; ++s) fl->idx[(f0 + r) * P + s] = Mp[r * p + s];
        }
        free(Mp);
        f0 += mp[p];
    }
    return 0;
}

static void feat_list_free(feat_list *fl)
{
    free(fl->deg); free(fl->idx); free(fl->cnt);
}

static double feat_value(const feat_list *fl, int64_t f, const double *x)
{
    double prod = 1.0;
    for (int s = 0; s < fl->deg[f]; ++s) prod *= x[fl->idx[f * fl->P + s]];
    return prod;
}

int64_t oracle_feature_dim(int dK, int P)
{
    int64_t M = 0;
    for (int p = 0; p < P; ++p) {
        int64_t m = oracle_tables(dK, p, NULL, NULL);
        if (m < 0) return -1;
        M += m;
    }
    return M;
}

/*
 * One head.  State S = sum_t phi(k_t) [v_t | 1]^T with the unweighted features of
 * all terms p < P stacked in table order; column dV is Z = sum_t phi(k_t)
 * ([TA Features]: Z_p and S_p and their recurrences).  After adding token T the
 * readout is y_T = (qw_T^T S)[:dV] / (qw_T^T S)[dV] with qw_T[f] = alpha_p C_p[f]
 * phi_p(q_T)[f]: both parts of the [TA Features] quotient carry the C_p-weighted
 * inner product and the alpha_p of the truncated kernel.
 *
 * q may be NULL (state only).  y (nullable, [n][dV]) receives the readout of every
 * row; S_out (nullable, [dV+1][M]) the state after the last token.  Returns M, or
 * -1 on failure.
 */
int64_t oracle_feature_form(const double *q, const double *k, const double *v,
                            int64_t n, int dK, int dV, int P,
                            double *y, double *S_out)
{
    feat_list fl;
    if (feat_list_build(dK, P, &fl) != 0) return -1;
    const int64_t M = fl.M;
    const int cols = dV + 1;
    double *S = (double *)calloc((size_t)(M * cols), sizeof(double));   /* [M][cols] */
    double *wq = (double *)malloc(sizeof(double) * (size_t)M);
    double *acc = (double *)malloc(sizeof(double) * (size_t)cols);
    if (!S || !wq || !acc) { feat_list_free(&fl); return -1; }
    double a[32];
    for (int p = 0; p < P; ++p) a[p] = alpha(p, dK);

    for (int64_t T = 0; T < n; ++T) {
        const double *kt = k + T * dK;
        const double *vt = v + T * dV;
#pragma omp parallel for schedule(static)
        for (int64_t f = 0; f < M; ++f) {
            double phik = feat_value(&fl, f, kt);
            for (int j = 0; j < dV; ++j) S[f * cols + j] += phik * vt[j];
            S[f * cols + dV] += phik;
        }
        if (y && q) {
            const double *qT = q + T * dK;
#pragma omp parallel for schedule(static)
            for (int64_t f = 0; f < M; ++f)
                wq[f] = a[fl.deg[f]] * (double)fl.cnt[f] * feat_value(&fl, f, qT);
#pragma omp parallel for schedule(static)
            for (int j = 0; j < cols; ++j) {
                double s = 0.0;
                for (int64_t f = 0; f < M; ++f) s += wq[f] * S[f * cols + j];
                acc[j] = s;
            }
            for (int j = 0; j < dV; ++j) y[T * dV + j] = acc[j] / acc[dV];
        }
    }
    if (S_out)
        for (int j = 0; j < cols; ++j)
            for (int64_t f = 0; f < M; ++f) S_out[j * M + f] = S[f * cols + j];
    free(S); free(wq); free(acc);
    feat_list_free(&fl);
    return M;
}

/*
 * Selected rows of the state of one head, summed over t < n:
 * S[f][j] = sum_t phi_f(k_t) u_t[j] with u_t = [v_t | 1], for the listed f only.
 * out: [nf][dV+1].  Used to check a few rows of a state too large to build whole.
 */
int oracle_state_rows(const double *k, const double *v, int64_t n, int dK, int dV,
                      int P, const int64_t *rows, int64_t nf, double *out)
{
    feat_list fl;
    if (feat_list_build(dK, P, &fl) != 0) return -1;
    const int cols = dV + 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nf; ++r) {
        int64_t f = rows[r];
        double *o = out + r * cols;
        for (int j = 0; j < cols; ++j) o[j] = 0.0;
        if (f < 0 || f >= fl.M) continue;
        for (int64_t t = 0; t < n; ++t) {
            double phik = feat_value(&fl, f, k + t * dK);
            for (int j = 0; j < dV; ++j) o[j] += phik * v[t * dV + j];
            o[dV] += phik;
        }
    }
    feat_list_free(&fl);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Exact softmax attention (the quantity the method approximates)             */
/* ------------------------------------------------------------------------- */

/*
 * y_T = sum_{t<=T} exp(q_T.k_t / c) v_t / sum_{t<=T} exp(q_T.k_t / c), c = sqrt(dK)
 * ([TA Taylor]: the exponential kernel being expanded).  The row maximum is
 * subtracted before exponentiating; it cancels in the quotient.  One row T of one
 * head (qh, kh: [n][dK], vh: [n][dV]).
 */
static void softmax_row(const double *qh, const double *kh, const double *vh, int64_t T,
                        int dK, int dV, double *yT)
{
    const double c = sqrt((double)dK);
    const double *qT = qh + T * dK;
    double mx = -INFINITY;
    for (int64_t t = 0; t <= T; ++t) {
        const double *kt = kh + t * dK;
        double x = 0.0;
        for (int i = 0; i < dK; ++i) x += qT[i] * kt[i];
        if (x / c > mx) mx = x / c;
    }
    double den = 0.0;
    for (int j = 0; j < dV; ++j) yT[j] = 0.0;
    for (int64_t t = 0; t <= T; ++t) {
        const double *kt = kh + t * dK;
        const double *vt = vh + t * dV;
        double x = 0.0;
        for (int i = 0; i < dK; ++i) x += qT[i] * kt[i];
        double e = exp(x / c - mx);
        den += e;
        for (int j = 0; j < dV; ++j) yT[j] += e * vt[j];
    }
    for (int j = 0; j < dV; ++j) yT[j] /= den;
}

/* Exact causal softmax attention of every row of every head. */
void oracle_softmax(const double *q, const double *k, const double *v,
                    int64_t heads, int64_t n, int dK, int dV, double *y)
{
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t h = 0; h < heads; ++h)
        for (int64_t T = 0; T < n; ++T)
            softmax_row(q + h * n * dK, k + h * n * dK, v + h * n * dV, T, dK, dV,
                        y + (h * n + T) * dV);
}

/* Sampled rows of the exact softmax attention: out[r] = y of token rows[r] of head
 * heads_of[r]; each row costs O(T (dK + dV)). */
void oracle_softmax_rows(const double *q, const double *k, const double *v,
                         int64_t n, int dK, int dV,
                         const int64_t *heads_of, const int64_t *rows, int64_t nr, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nr; ++r) {
        const int64_t h = heads_of[r];
        softmax_row(q + h * n * dK, k + h * n * dK, v + h * n * dV, rows[r], dK, dV,
                    out + r * dV);
    }
}

/* Number of OpenMP threads the oracle runs with (for the benchmark report). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
