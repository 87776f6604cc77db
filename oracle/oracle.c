/*
 * oracle.c -- plain CPU reference for Entwine's GEMM-ReduceScatter, taken at
 * one rank's share of the work.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header, table or helper with the
 * HIP library; it is built with gcc on its own.
 *
 * Source: "Entwine: Coordinating Tiled Computation and Fine-Grained
 * Communication across GPUs" (paperpeel.com/paper/2609.11562).
 *   - Sec. 2.1 (GEMM-ReduceScatter Execution): with W ranks, rank r holds a
 *     slice of the reduction dimension and computes a full-size partial
 *     product; the ReduceScatter sums the partials and gives each rank one
 *     contiguous row partition of the sum.
 *   - Sec. 3.1 (Coordinating Tiled Computation and Communication): the
 *     destination rank d forms its output from the contributions V[r,d,.]
 *     of every source rank r, its own included.
 *   - Sec. 4.2 (Producer Traversal, Publication, and Reduction), ReduceTile:
 *     the accumulator starts from the local contribution and the peers'
 *     values are added in rank order.
 *   - Sec. 5.2.2 (Layer-Level Performance): the layer chain continues the
 *     ReduceScatter with a residual addition and an RMSNorm.
 *
 * Everything here is evaluated in fp64 from the exact values that the device
 * receives (bf16 or fp32 inputs widened exactly), with plain loops and no
 * blocking.  The single fp32 routine, oracle_reduce_f32, is the closed form
 * of the reduction step carried out in fp32 in the rank order above and
 * rounded to the output type; it is what a bit-exact comparison of the
 * reduction uses.
 *
 * Layout conventions (all row-major, element counts, no padding):
 *   X  [M][K] bf16 bits                       -- this rank's reduction slice
 *   W  [N][K] bf16 bits  (ORACLE_W_NK)        -- K contiguous, or
 *      [K][N] bf16 bits  (ORACLE_W_KN)        -- N contiguous
 *   peers[r] [M/P][N] bf16 bits or fp32       -- V[r, rank, .]; peers[rank] unused
 *   out  [rows][N] double                     -- rows [row_begin,row_end) of the
 *                                                rank's partition
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_W_NK 0
#define ORACLE_W_KN 1
#define ORACLE_BF16 0
#define ORACLE_F32 1

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 3

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double widen_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    return widen_bf16(((const uint16_t *)base)[idx]);
}

int oracle_num_threads(int threads)
{
    if (threads > 0)
        return threads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/* ---------------------------------------------------------------------- */
/* Partial product C = X[rows] * W in fp64.                                */
/* ---------------------------------------------------------------------- */

typedef struct {
    const double *Xd;   /* widened X rows [row_begin,row_end) x K */
    const double *Wd;   /* widened W, same layout as given          */
    int w_layout;
    int64_t N, K;
    int64_t i_begin, i_end; /* local row range of this worker        */
    double *C;          /* [(row_end-row_begin)][N]                  */
} gemm_job;

static void *gemm_worker(void *arg)
{
    gemm_job *g = (gemm_job *)arg;
    const int64_t N = g->N, K = g->K;
    for (int64_t i = g->i_begin; i < g->i_end; ++i) {
        const double *x = g->Xd + i * K;
        double *c = g->C + i * N;
        if (g->w_layout == ORACLE_W_KN) {
            /* C[i][j] = sum_k X[i][k] * W[k][j], k outer so W rows stream. */
            for (int64_t j = 0; j < N; ++j)
                c[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double xv = x[k];
                const double *w = g->Wd + k * N;
                for (int64_t j = 0; j < N; ++j)
                    c[j] += xv * w[j];
            }
        } else {
            /* C[i][j] = sum_k X[i][k] * W[j][k] (W given as [N][K]). */
            for (int64_t j = 0; j < N; ++j) {
                const double *w = g->Wd + j * K;
                double s = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    s += x[k] * w[k];
                c[j] = s;
            }
        }
    }
    return NULL;
}

/*
 * C[(i - row_begin)][j] = sum_{k<K} X[i][k] * W(k, j)  for row_begin <= i < row_end.
 * This is the rank's partial contribution (Sec. 2.1) restricted to a row range.
 */
int oracle_partial_gemm(const uint16_t *X, const uint16_t *W, int w_layout,
                        int64_t M, int64_t N, int64_t K,
                        int64_t row_begin, int64_t row_end, int threads,
                        double *C)
{
    if (!X || !W || !C || M <= 0 || N <= 0 || K <= 0 || row_begin < 0 ||
        row_end > M || row_begin > row_end ||
        (w_layout != ORACLE_W_NK && w_layout != ORACLE_W_KN))
        return ORACLE_EINVAL;
    const int64_t rows = row_end - row_begin;
    if (rows == 0)
        return ORACLE_OK;

    double *Xd = (double *)malloc((size_t)(rows * K) * sizeof(double));
    double *Wd = (double *)malloc((size_t)(N * K) * sizeof(double));
    if (!Xd || !Wd) {
        free(Xd);
        free(Wd);
        return ORACLE_ENOMEM;
    }
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t k = 0; k < K; ++k)
            Xd[i * K + k] = widen_bf16(X[(row_begin + i) * K + k]);
    for (int64_t e = 0; e < N * K; ++e)
        Wd[e] = widen_bf16(W[e]);

    int nt = oracle_num_threads(threads);
    if (nt > rows)
        nt = (int)rows;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    gemm_job *jobs = (gemm_job *)malloc(sizeof(gemm_job) * (size_t)nt);
    if (!tid || !jobs) {
        free(Xd); free(Wd); free(tid); free(jobs);
        return ORACLE_ENOMEM;
    }
    int launched = 0;
    for (int t = 0; t < nt; ++t) {
        jobs[t].Xd = Xd;
        jobs[t].Wd = Wd;
        jobs[t].w_layout = w_layout;
        jobs[t].N = N;
        jobs[t].K = K;
        jobs[t].i_begin = rows * t / nt;
        jobs[t].i_end = rows * (t + 1) / nt;
        jobs[t].C = C;
        if (t > 0 && pthread_create(&tid[t], NULL, gemm_worker, &jobs[t]) == 0) {
            ++launched;
        } else if (t > 0) {
            gemm_worker(&jobs[t]); /* no thread available: run inline */
            tid[t] = (pthread_t)0;
        }
    }
    gemm_worker(&jobs[0]);
    for (int t = 1; t < nt; ++t)
        if (tid[t] != (pthread_t)0)
            pthread_join(tid[t], NULL);
    (void)launched;
    free(Xd); free(Wd); free(tid); free(jobs);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* The operation: this rank's row partition of the reduce-scattered sum.   */
/* ---------------------------------------------------------------------- */

/*
 * For simulated rank d = `rank` with partition rows R = M/P:
 *   out[i - row_begin][j] = C_d[d*R + i][j] + sum_{r != d, r ascending} V_r[i][j]
 * for row_begin <= i < row_end <= R, all j < N, where C_d = X * W over this
 * rank's reduction slice (Sec. 2.1) and V_r = peers[r] is peer r's
 * contribution to partition d (Sec. 3.1).  The local contribution is the
 * starting value and peers follow in ascending rank order (Sec. 4.2,
 * ReduceTile); in fp64 the order only matters at the last few bits.
 */
int oracle_gemm_rs(const uint16_t *X, const uint16_t *W, int w_layout,
                   const void *const *peers, int peer_dtype,
                   int64_t M, int64_t N, int64_t K, int P, int rank,
                   int64_t row_begin, int64_t row_end, int threads,
                   double *out)
{
    if (P < 1 || rank < 0 || rank >= P || M % P != 0 ||
        (peer_dtype != ORACLE_BF16 && peer_dtype != ORACLE_F32))
        return ORACLE_EINVAL;
    const int64_t R = M / P;
    if (row_begin < 0 || row_end > R || row_begin > row_end)
        return ORACLE_EINVAL;
    for (int r = 0; r < P; ++r)
        if (r != rank && !peers[r])
            return ORACLE_EINVAL;

    int rc = oracle_partial_gemm(X, W, w_layout, M, N, K,
                                 (int64_t)rank * R + row_begin,
                                 (int64_t)rank * R + row_end, threads, out);
    if (rc != ORACLE_OK)
        return rc;

    for (int64_t i = row_begin; i < row_end; ++i) {
        double *o = out + (i - row_begin) * N;
        for (int r = 0; r < P; ++r) {
            if (r == rank)
                continue;
            for (int64_t j = 0; j < N; ++j)
                o[j] += load_elem(peers[r], peer_dtype, i * N + j);
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* The reduction step in fp32, bit for bit.                                 */
/* ---------------------------------------------------------------------- */

/* binary32 -> bf16 with round-to-nearest-even; NaN stays NaN (quiet). */
static uint16_t round_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/*
 * The ReduceTile closed form (Sec. 4.2) evaluated in binary32:
 *   acc = own[e];  for r ascending, r != rank: acc = fl32(acc + V_r[e]);
 *   with a residual (the layer chain of Sec. 5.2.2, added as one more term
 *   after the peers): acc = fl32(acc + residual[e]);
 *   out[e] = acc rounded to out_dtype (bf16 with round-to-nearest-even, or
 *            fp32 unchanged).
 * `own` is the rank's own fp32 partial for its partition ([rows][N]);
 * `residual` is NULL or [rows][N] in res_dtype.
 */
int oracle_reduce_f32(const float *own, const void *const *peers, int peer_dtype,
                      int P, int rank, int64_t rows, int64_t N, const void *residual,
                      int res_dtype, int out_dtype, void *out)
{
    if (!own || !out || P < 1 || rank < 0 || rank >= P || rows < 0 || N < 0 ||
        (peer_dtype != ORACLE_BF16 && peer_dtype != ORACLE_F32) ||
        (res_dtype != ORACLE_BF16 && res_dtype != ORACLE_F32) ||
        (out_dtype != ORACLE_BF16 && out_dtype != ORACLE_F32))
        return ORACLE_EINVAL;
    for (int r = 0; r < P; ++r)
        if (r != rank && !peers[r])
            return ORACLE_EINVAL;
    for (int64_t e = 0; e < rows * N; ++e) {
        float acc = own[e];
        for (int r = 0; r < P; ++r) {
            if (r == rank)
                continue;
            float v = (float)load_elem(peers[r], peer_dtype, e);
            acc = acc + v;
        }
        if (residual)
            acc = acc + (float)load_elem(residual, res_dtype, e);
        if (out_dtype == ORACLE_BF16)
            ((uint16_t *)out)[e] = round_to_bf16(acc);
        else
            ((float *)out)[e] = acc;
    }
    return ORACLE_OK;
}

/*
 * RMSNorm of each row (Sec. 5.2.2: the layer chain's normalization after the
 * residual addition), in fp64 from the stored values h:
 *   ms_i = (1/N) * sum_j h[i][j]^2
 *   y[i][j] = gamma[j] * h[i][j] / sqrt(ms_i + eps)
 * h is [rows][N] and gamma [N], each bf16 bits or fp32; y is [rows][N] double.
 */
int oracle_rmsnorm(const void *h, int h_dtype, const void *gamma, int g_dtype, double eps,
                   int64_t rows, int64_t N, double *y)
{
    if (!h || !gamma || !y || rows < 0 || N <= 0 || !(eps >= 0.0) ||
        (h_dtype != ORACLE_BF16 && h_dtype != ORACLE_F32) ||
        (g_dtype != ORACLE_BF16 && g_dtype != ORACLE_F32))
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < rows; ++i) {
        double ss = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double v = load_elem(h, h_dtype, i * N + j);
            ss += v * v;
        }
        double scale = 1.0 / sqrt(ss / (double)N + eps);
        for (int64_t j = 0; j < N; ++j)
            y[i * N + j] = load_elem(gamma, g_dtype, j) * load_elem(h, h_dtype, i * N + j) * scale;
    }
    return ORACLE_OK;
}
