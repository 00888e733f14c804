/*
 * Soft-DTW oracle: a plain, slow, fp64 CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library and must never be used as a
 * fallback for it.
 *
 * What it computes (sources):
 *  - Soft-DTW of Cuturi & Blondel, "Soft-DTW: a Differentiable Loss Function
 *    for Time-Series" (ICML 2017), which the README "SoftDTW-CUDA (PyTorch +
 *    Numba)" credits in its "Acknowledgments" section.  The pages do not
 *    print the recurrence; it is taken in its textbook form:
 *      R[0,0] = 0, R[i,0] = R[0,j] = +inf (i,j >= 1),
 *      R[i,j] = Dist[i-1,j-1] + softmin_g(R[i-1,j-1], R[i-1,j], R[i,j-1]),
 *      softmin_g(a) = -g * log(sum_k exp(-a_k / g)),
 *      loss = R[N,M].
 *  - Dist is the squared Euclidean distance ("Usage", dist="sqeuclidean";
 *    "Notes": squared Euclidean distances are never negative).
 *  - The backward pass follows the review page "SoftDTW-CUDA-Torch:
 *    Memory-Efficient GPU-Accelerated Soft Dynamic Time Warping for PyTorch",
 *    section "Proposed method": a log-space backward recursion driven by
 *    logsumexp, with the exponential taken only after the recursion ends.
 *    In Cuturi & Blondel's notation the alignment matrix satisfies
 *      E[N,M] = 1,
 *      E[i,j] = sum over in-grid successors s of (i,j) of
 *               E[s] * exp((R[s] - Dist_s - R[i,j]) / g),
 *    so G = log E obeys G[N,M] = 0 and
 *      G[i,j] = LSE_s (G[s] + (R[s] - Dist_s - R[i,j]) / g).
 *  - The chain rule through Dist = ||x_i - y_j||^2:
 *      dL/dx_i = 2 gl * sum_j E[i,j] (x_i - y_j),
 *      dL/dy_j = 2 gl * sum_i E[i,j] (y_j - x_i),
 *    where gl is the upstream gradient of this pair's loss.
 *
 * Conventions: arrays are row-major and contiguous.  Per pair, R and G are
 * (N+1) x (M+1) with the DP cell (i,j), 1 <= i <= N, 1 <= j <= M, at
 * [i*(M+1)+j]; Dist and E are N x M with the cell (i,j) at [(i-1)*M+(j-1)].
 * Everything is IEEE fp64 and uses libm exp/log.  Batched entry points loop
 * over the B pairs with OpenMP; a pair is computed by one thread in the
 * plain row-major order, so results do not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_INF (1.0 / 0.0)

/* softmin_g over three values; +inf entries contribute exp(-inf) = 0. */
static double orc_softmin3(double a, double b, double c, double g)
{
    double m = a;
    if (b < m) m = b;
    if (c < m) m = c;
    if (m == ORC_INF) return ORC_INF;
    double s = exp(-(a - m) / g) + exp(-(b - m) / g) + exp(-(c - m) / g);
    return m - g * log(s);
}

/* Squared Euclidean distance, direct form sum_d (x_d - y_d)^2, in fp64 from
 * fp32 inputs (the difference and the square of fp32 values are exact in
 * fp64; only the summation rounds). */
void oracle_sqeuclid(const float *x, const float *y, int64_t B, int64_t N,
                     int64_t M, int64_t D, double *dist)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        const float *xb = x + b * N * D;
        const float *yb = y + b * M * D;
        double *db = dist + b * N * M;
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = 0; j < M; ++j) {
                double s = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    double t = (double)xb[i * D + d] - (double)yb[j * D + d];
                    s += t * t;
                }
                db[i * M + j] = s;
            }
    }
}

/* One pair: the forward recurrence.  R has (N+1)*(M+1) entries. */
static double orc_forward_pair(const double *dist, int64_t N, int64_t M,
                               double g, double *R)
{
    const int64_t W = M + 1;
    R[0] = 0.0;
    for (int64_t j = 1; j <= M; ++j) R[j] = ORC_INF;
    for (int64_t i = 1; i <= N; ++i) {
        R[i * W] = ORC_INF;
        for (int64_t j = 1; j <= M; ++j) {
            double sm = orc_softmin3(R[(i - 1) * W + (j - 1)],
                                     R[(i - 1) * W + j],
                                     R[i * W + (j - 1)], g);
            R[i * W + j] = dist[(i - 1) * M + (j - 1)] + sm;
        }
    }
    return R[N * W + M];
}

/* Batched forward: loss[b] = R_b[N,M].  R (optional) receives every pair's
 * (N+1)x(M+1) table; when NULL a per-thread scratch table is used. */
int oracle_sdtw_forward(const double *dist, int64_t B, int64_t N, int64_t M,
                        double gamma, double *R, double *loss)
{
    const int64_t cells = (N + 1) * (M + 1);
    int err = 0;
#pragma omp parallel
    {
        double *scratch = NULL;
        if (!R) {
            scratch = (double *)malloc(sizeof(double) * (size_t)cells);
            if (!scratch) {
#pragma omp atomic write
                err = 1;
            }
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < B; ++b) {
            double *Rb = R ? R + b * cells : scratch;
            if (!Rb) continue;
            loss[b] = orc_forward_pair(dist + b * N * M, N, M, gamma, Rb);
        }
        free(scratch);
    }
    return err;
}

/* One pair: the log-space backward in the textbook form.  G has
 * (N+1)*(M+1) entries (row 0 and column 0 unused); E is N x M. */
static void orc_backward_pair(const double *dist, const double *R, int64_t N,
                              int64_t M, double g, double *G, double *E)
{
    const int64_t W = M + 1;
    for (int64_t i = N; i >= 1; --i) {
        for (int64_t j = M; j >= 1; --j) {
            if (i == N && j == M) {
                G[i * W + j] = 0.0;
                continue;
            }
            const double r = R[i * W + j];
            double t[3] = {-ORC_INF, -ORC_INF, -ORC_INF};
            int n = 0;
            if (i < N) /* successor (i+1, j) */
                t[n++] = G[(i + 1) * W + j] +
                         (R[(i + 1) * W + j] - dist[i * M + (j - 1)] - r) / g;
            if (j < M) /* successor (i, j+1) */
                t[n++] = G[i * W + (j + 1)] +
                         (R[i * W + (j + 1)] - dist[(i - 1) * M + j] - r) / g;
            if (i < N && j < M) /* successor (i+1, j+1) */
                t[n++] = G[(i + 1) * W + (j + 1)] +
                         (R[(i + 1) * W + (j + 1)] - dist[i * M + j] - r) / g;
            double mx = t[0];
            for (int k = 1; k < n; ++k)
                if (t[k] > mx) mx = t[k];
            double s = 0.0;
            if (mx == -ORC_INF) {
                G[i * W + j] = -ORC_INF;
                continue;
            }
            for (int k = 0; k < n; ++k) s += exp(t[k] - mx);
            G[i * W + j] = mx + log(s);
        }
    }
    /* The exponential is applied once the recursion is complete. */
    for (int64_t i = 1; i <= N; ++i)
        for (int64_t j = 1; j <= M; ++j)
            E[(i - 1) * M + (j - 1)] = exp(G[i * W + j]);
}

/* Batched backward from stored R tables: E is B x N x M. */
int oracle_sdtw_backward(const double *dist, const double *R, int64_t B,
                         int64_t N, int64_t M, double gamma, double *E)
{
    const int64_t cells = (N + 1) * (M + 1);
    int err = 0;
#pragma omp parallel
    {
        double *G = (double *)malloc(sizeof(double) * (size_t)cells);
        if (!G) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < B; ++b) {
            if (!G) continue;
            orc_backward_pair(dist + b * N * M, R + b * cells, N, M, gamma, G,
                              E + b * N * M);
        }
        free(G);
    }
    return err;
}

/* A second, independent backward with the same mathematics, used only to
 * cross-check the first: every successor s re-derives its own softmin weights
 * from its three predecessors' R values,
 *   w(p -> s) = exp(-(R[p] - m_s)/g) / sum_q exp(-(R[q] - m_s)/g),
 * (m_s = min over the predecessors q of s) and E is propagated in the linear
 * domain, E[p] = sum_s w(p -> s) E[s].  It never reads Dist. */
int oracle_sdtw_backward_local(const double *R, int64_t B, int64_t N,
                               int64_t M, double gamma, double *E)
{
    const int64_t W = M + 1;
    const int64_t cells = (N + 1) * W;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        const double *Rb = R + b * cells;
        double *Eb = E + b * N * M;
        for (int64_t i = N; i >= 1; --i)
            for (int64_t j = M; j >= 1; --j) {
                if (i == N && j == M) {
                    Eb[(i - 1) * M + (j - 1)] = 1.0;
                    continue;
                }
                double acc = 0.0;
                const int64_t si[3] = {i + 1, i, i + 1};
                const int64_t sj[3] = {j, j + 1, j + 1};
                for (int k = 0; k < 3; ++k) {
                    const int64_t a = si[k], c = sj[k];
                    if (a > N || c > M) continue;
                    const double pa = Rb[(a - 1) * W + (c - 1)];
                    const double pb = Rb[(a - 1) * W + c];
                    const double pc = Rb[a * W + (c - 1)];
                    double m = pa;
                    if (pb < m) m = pb;
                    if (pc < m) m = pc;
                    const double z = exp(-(pa - m) / gamma) +
                                     exp(-(pb - m) / gamma) +
                                     exp(-(pc - m) / gamma);
                    const double w = exp(-(Rb[i * W + j] - m) / gamma) / z;
                    acc += w * Eb[(a - 1) * M + (c - 1)];
                }
                Eb[(i - 1) * M + (j - 1)] = acc;
            }
    }
    return 0;
}

/* Chain rule through the squared Euclidean distance, per pair b with the
 * upstream gradient gl[b].  gx is B x N x D, gy is B x M x D (fp64). */
void oracle_sqeuclid_vjp(const float *x, const float *y, const double *E,
                         const double *gl, int64_t B, int64_t N, int64_t M,
                         int64_t D, double *gx, double *gy)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        const float *xb = x + b * N * D;
        const float *yb = y + b * M * D;
        const double *Eb = E + b * N * M;
        double *gxb = gx + b * N * D;
        double *gyb = gy + b * M * D;
        for (int64_t k = 0; k < N * D; ++k) gxb[k] = 0.0;
        for (int64_t k = 0; k < M * D; ++k) gyb[k] = 0.0;
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = 0; j < M; ++j) {
                const double e = Eb[i * M + j];
                for (int64_t d = 0; d < D; ++d) {
                    const double t = (double)xb[i * D + d] - (double)yb[j * D + d];
                    gxb[i * D + d] += e * t;
                    gyb[j * D + d] -= e * t;
                }
            }
        const double s = 2.0 * gl[b];
        for (int64_t k = 0; k < N * D; ++k) gxb[k] *= s;
        for (int64_t k = 0; k < M * D; ++k) gyb[k] *= s;
    }
}

/* Everything for a batch with bounded memory: for each pair, Dist (exact
 * fp64, optionally rounded to fp32 first when round_dist_f32 != 0), the
 * forward, the textbook backward and the chain rule, using per-thread
 * scratch of about 3 (N+1)(M+1) doubles.  E_out (B x N x M) is optional. */
int oracle_sdtw_value_and_grad(const float *x, const float *y, int64_t B,
                               int64_t N, int64_t M, int64_t D, double gamma,
                               int round_dist_f32, const double *gl,
                               double *loss, double *gx, double *gy,
                               double *E_out)
{
    const int64_t cells = (N + 1) * (M + 1);
    int err = 0;
#pragma omp parallel
    {
        double *dist = (double *)malloc(sizeof(double) * (size_t)(N * M));
        double *R = (double *)malloc(sizeof(double) * (size_t)cells);
        double *G = (double *)malloc(sizeof(double) * (size_t)cells);
        double *E = (double *)malloc(sizeof(double) * (size_t)(N * M));
        if (!dist || !R || !G || !E) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < B; ++b) {
            if (!dist || !R || !G || !E) continue;
            const float *xb = x + b * N * D;
            const float *yb = y + b * M * D;
            for (int64_t i = 0; i < N; ++i)
                for (int64_t j = 0; j < M; ++j) {
                    double s = 0.0;
                    for (int64_t d = 0; d < D; ++d) {
                        double t = (double)xb[i * D + d] - (double)yb[j * D + d];
                        s += t * t;
                    }
                    if (round_dist_f32) s = (double)(float)s;
                    dist[i * M + j] = s;
                }
            loss[b] = orc_forward_pair(dist, N, M, gamma, R);
            orc_backward_pair(dist, R, N, M, gamma, G, E);
            double *gxb = gx + b * N * D;
            double *gyb = gy + b * M * D;
            for (int64_t k = 0; k < N * D; ++k) gxb[k] = 0.0;
            for (int64_t k = 0; k < M * D; ++k) gyb[k] = 0.0;
            for (int64_t i = 0; i < N; ++i)
                for (int64_t j = 0; j < M; ++j) {
                    const double e = E[i * M + j];
                    for (int64_t d = 0; d < D; ++d) {
                        const double t = (double)xb[i * D + d] - (double)yb[j * D + d];
                        gxb[i * D + d] += e * t;
                        gyb[j * D + d] -= e * t;
                    }
                }
            const double sc = 2.0 * gl[b];
            for (int64_t k = 0; k < N * D; ++k) gxb[k] *= sc;
            for (int64_t k = 0; k < M * D; ++k) gyb[k] *= sc;
            if (E_out)
                for (int64_t k = 0; k < N * M; ++k) E_out[b * N * M + k] = E[k];
        }
        free(dist);
        free(R);
        free(G);
        free(E);
    }
    return err;
}

/* Hard DTW (the g -> 0 limit): the same recurrence with min. */
int oracle_dtw(const double *dist, int64_t B, int64_t N, int64_t M,
               double *out)
{
    const int64_t W = M + 1;
    int err = 0;
#pragma omp parallel
    {
        double *R = (double *)malloc(sizeof(double) * (size_t)((N + 1) * W));
        if (!R) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < B; ++b) {
            if (!R) continue;
            const double *db = dist + b * N * M;
            R[0] = 0.0;
            for (int64_t j = 1; j <= M; ++j) R[j] = ORC_INF;
            for (int64_t i = 1; i <= N; ++i) {
                R[i * W] = ORC_INF;
                for (int64_t j = 1; j <= M; ++j) {
                    double m = R[(i - 1) * W + (j - 1)];
                    if (R[(i - 1) * W + j] < m) m = R[(i - 1) * W + j];
                    if (R[i * W + (j - 1)] < m) m = R[i * W + (j - 1)];
                    R[i * W + j] = db[(i - 1) * M + (j - 1)] + m;
                }
            }
            out[b] = R[N * W + M];
        }
        free(R);
    }
    return err;
}

/* Sets the thread count of the OpenMP regions that follow (timing the
 * oracle on a chosen number of cores); n < 1 is ignored. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
