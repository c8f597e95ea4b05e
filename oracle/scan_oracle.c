/*
 * fp64 CPU oracle of the Mamba selective-scan forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file:
 * only the tests, the smoke check and the bench's CPU-baseline leg use it. It shares no code,
 * header, table or helper with the HIP library.
 *
 * It is the plain sequential recurrence, in the order and notation of the pages:
 *   - "Mamba代码实战：手把手教你用PyTorch复现选择性扫描核心逻辑（附避坑指南）"
 *       §2.1 layouts: u, delta, z (batch, D, L); A (D, N); B, C (batch, N, L); D, delta_bias (D);
 *       §2.2 / §6 delta preprocessing: delta + delta_bias[d], then softplus (flag set) or exp;
 *       §3.1 discretisation: dA = exp(delta * A[d, n]),  dB = delta * B[b, n, t];
 *       §3.2 recurrence from a zero state: h = dA * h + dB * u, per step, with an output per step;
 *       §3.3 skip and gate: y += u * D[d], then y *= silu(z);
 *       §6 return value: (y, state after the last step).
 *   - "Mamba-minimal项目解析：深入理解Mamba模型的极简实现", "关键技术点 1. 选择性扫描算法": the output
 *       contraction y[b, d, t] = sum_n h[b, d, n] * C[b, n, t] (the subscripts there are right;
 *       the first page's 'bdn,bdn->bd' label on C is a slip).
 *   - The initial state h0 (NULL = zeros) follows the scan of "手把手用PyTorch实现Mamba的SSM层
 *       从HiPPO矩阵到选择性扫描算法", §3.1, which takes the state h as an argument.
 * softplus(x) = ln(1 + e^x) exactly (beta 1, no linearisation threshold), evaluated as
 * max(x, 0) + log1p(exp(-|x|)), which is the same function. silu(z) = z / (1 + e^-z).
 * No clamp of delta, no special handling of overflow: fp64 libm exp/log1p throughout.
 *
 * Inputs are contiguous. bf16 inputs arrive as their 16-bit patterns and are widened here
 * (exactly: the pattern is the high half of an fp32), fp32 inputs are widened to fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

typedef struct {
    int64_t batch, dim, len, dstate;
    int in_dtype;
    const void *u, *delta, *z, *B, *C;
    const float *A, *Dvec, *delta_bias;
    const double* h0;
    int delta_softplus;
    int zoh_b;
    const int64_t* rows;
    int64_t nrows;
    double *y, *last_state;
} orc_args;

static double widen(const void* p, int in_dtype, int64_t i) {
    if (in_dtype == ORC_F32) return (double)((const float*)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Zero-order-hold input coefficient of one diagonal state: B_d = A^-1 (e^{A dt} - 1) B, written
 * per state as (e^{A dt} - 1) / A ("手把手用PyTorch实现Mamba的SSM层…" §2.1); at A = 0 (not
 * invertible) its limit dt. expm1 keeps it accurate when A dt is small. */
static double zoh_coef(double dt, double An) { return An == 0.0 ? dt : expm1(dt * An) / An; }

/* Its derivative with respect to A: d/dA [(e^{A dt} - 1) / A] = (dt e^{A dt} - (e^{A dt} - 1)/A) / A,
 * whose limit at A = 0 is dt^2 / 2. For |A dt| < 1/64 the Taylor series of the same function,
 * dt^2 (1/2 + x/3 + x^2/8 + x^3/30 + x^4/144) with x = A dt (the first dropped term, x^5 / 840,
 * is below 3e-12 of the sum there), so that the difference of two nearly equal terms is never
 * formed; above it the closed form, whose cancellation costs at most a factor 2/|x| < 128 on the
 * fp64 rounding. Its derivative with respect to dt is e^{A dt}. */
static double zoh_coef_dA(double dt, double An) {
    const double x = dt * An;
    if (fabs(x) < 1.0 / 64.0)
        return dt * dt * (0.5 + x * (1.0 / 3.0 + x * (1.0 / 8.0 + x * (1.0 / 30.0 + x / 144.0))));
    return (dt * exp(x) - expm1(x) / An) / An;
}

/* One row (b, d): writes y[out_row, 0..L) and last_state[out_row, 0..N). */
static void scan_row(const orc_args* a, int64_t b, int64_t d, int64_t out_row, double* h) {
    const int64_t L = a->len, N = a->dstate, D = a->dim;
    const int64_t row_off = (b * D + d) * L;  /* u, delta, z (batch, D, L) */
    const int64_t bc_off = b * N * L;         /* B, C (batch, N, L) */
    for (int64_t n = 0; n < N; ++n) h[n] = a->h0 ? a->h0[(b * D + d) * N + n] : 0.0;
    const double bias = a->delta_bias ? (double)a->delta_bias[d] : 0.0;
    const double dskip = a->Dvec ? (double)a->Dvec[d] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const double x = widen(a->delta, a->in_dtype, row_off + t) + bias;
        const double dt = a->delta_softplus ? softplus(x) : exp(x);
        const double ut = widen(a->u, a->in_dtype, row_off + t);
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double Bt = widen(a->B, a->in_dtype, bc_off + n * L + t);
            const double Ct = widen(a->C, a->in_dtype, bc_off + n * L + t);
            const double An = (double)a->A[d * N + n];
            const double dA = exp(dt * An);
            const double dB = a->zoh_b ? zoh_coef(dt, An) : dt; /* discretised B per unit B */
            h[n] = dA * h[n] + dB * Bt * ut;
            acc += Ct * h[n];
        }
        double v = acc + dskip * ut;
        if (a->z) v *= silu(widen(a->z, a->in_dtype, row_off + t));
        a->y[out_row * L + t] = v;
    }
    if (a->last_state)
        for (int64_t n = 0; n < N; ++n) a->last_state[out_row * N + n] = h[n];
}

typedef struct {
    const orc_args* a;
    int64_t begin, end;
} orc_job;

static void* orc_worker(void* p) {
    const orc_job* j = (const orc_job*)p;
    double* h = (double*)malloc(sizeof(double) * (size_t)(j->a->dstate > 0 ? j->a->dstate : 1));
    if (!h) return (void*)1;
    for (int64_t k = j->begin; k < j->end; ++k) {
        const int64_t flat = j->a->rows ? j->a->rows[k] : k;
        scan_row(j->a, flat / j->a->dim, flat % j->a->dim, k, h);
    }
    free(h);
    return NULL;
}

#define ORC_MAX_THREADS 256

/*
 * Compute rows of the scan.  rows == NULL: all batch*dim rows in order (nrows ignored);
 * otherwise the listed flat rows b*dim + d.  y is (nrows, L) fp64, last_state (nrows, N) fp64 or
 * NULL.  z, Dvec, delta_bias, h0 may be NULL (absent).  h0 is (batch, dim, N) fp64, so that a
 * scan split at any step continues exactly from the fp64 state of its first part.
 * Returns 0, or a negative value on a bad argument or allocation failure.
 */
int oracle_selective_scan_ex(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int in_dtype,
                             const void* u, const void* delta, const void* z, const void* B,
                             const void* C, const float* A, const float* Dvec,
                             const float* delta_bias, const double* h0, int delta_softplus,
                             int zoh_b, const int64_t* rows, int64_t nrows, double* y,
                             double* last_state, int nthreads) {
    if (batch <= 0 || dim <= 0 || len <= 0 || dstate <= 0) return -2;
    if (in_dtype != ORC_F32 && in_dtype != ORC_BF16) return -4;
    if (!u || !delta || !B || !C || !A || !y) return -1;
    orc_args a = {batch, dim, len, dstate, in_dtype, u, delta, z, B, C, A, Dvec, delta_bias, h0,
                  delta_softplus, zoh_b, rows, rows ? nrows : batch * dim, y, last_state};
    if (rows)
        for (int64_t k = 0; k < nrows; ++k)
            if (rows[k] < 0 || rows[k] >= batch * dim) return -2;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > ORC_MAX_THREADS) nthreads = ORC_MAX_THREADS;
    if (nthreads > a.nrows) nthreads = (int)a.nrows;
    orc_job jobs[ORC_MAX_THREADS];
    pthread_t tids[ORC_MAX_THREADS];
    const int64_t per = (a.nrows + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].a = &a;
        jobs[t].begin = per * t < a.nrows ? per * t : a.nrows;
        jobs[t].end = per * (t + 1) < a.nrows ? per * (t + 1) : a.nrows;
    }
    int ok = 1;
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, orc_worker, &jobs[t]) != 0) break;
        started = t;
    }
    if (orc_worker(&jobs[0]) != NULL) ok = 0;
    for (int t = 1; t <= started; ++t) {
        void* r = NULL;
        pthread_join(tids[t], &r);
        if (r != NULL) ok = 0;
    }
    for (int t = started + 1; t < nthreads; ++t)
        if (orc_worker(&jobs[t]) != NULL) ok = 0;
    return ok ? 0 : -8;
}

/* The scan with Euler B (dB = dt B), as the pages' selective scan computes it. */
int oracle_selective_scan(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int in_dtype,
                          const void* u, const void* delta, const void* z, const void* B,
                          const void* C, const float* A, const float* Dvec,
                          const float* delta_bias, const double* h0, int delta_softplus,
                          const int64_t* rows, int64_t nrows, double* y, double* last_state,
                          int nthreads) {
    return oracle_selective_scan_ex(batch, dim, len, dstate, in_dtype, u, delta, z, B, C, A, Dvec,
                                    delta_bias, h0, delta_softplus, 0, rows, nrows, y, last_state,
                                    nthreads);
}

/* ----------------------------------------------------------------------------------------------
 * Backward pass: the gradients of a scalar loss that depends on the scan through y (gradient gy,
 * (batch, D, L)) and through the final state (gradient glast, (batch, D, N), or none).
 *
 * Training is what "手把手用PyTorch实现Mamba的SSM层…" §4.2 (memory-efficient training: states are
 * not kept from the forward pass but recomputed for the backward) and "Mamba代码实战…" §7 (item 3,
 * an efficient backward pass by automatic differentiation) ask of the scan. The derivative has a
 * plain definition; this is it written out by the chain rule through the forward recurrence
 * above, taken in reverse step order. With x = delta + bias, dt = softplus(x) (or exp(x)),
 * a_n = exp(dt A[d,n]), h_t = a h_{t-1} + dt B_t u_t, p_t = sum_n C_t h_t + D u_t, y_t = p_t g_t,
 * g_t = silu(z_t) (1 without z), and lam_t = dLoss/dh_t (lam after the last step = glast):
 *   gp_t = gy_t g_t;  gz_t = gy_t p_t silu'(z_t);  lam_t += gp_t C_t
 *   gC[b,n,t] += gp_t h_t;  gB[b,n,t] += lam_t dt_t u_t  (summed over d)
 *   gu_t = gp_t D + sum_n lam_t dt_t B_t
 *   gdt_t = sum_n lam_t (a_t h_{t-1} A + B_t u_t);  gA[d,n] += lam_t a_t h_{t-1} dt_t (summed over b, t)
 *   gx_t = gdt_t sigmoid(x_t) (softplus) or gdt_t dt_t (exp);  gdelta_t = gx_t;  gbias[d] += gx_t
 *   gD[d] += gp_t u_t;  then lam_{t-1} = a_t lam_t;  gh0 = lam before the first step.
 * With the zero-order hold the input term is c_t B_t u_t with c_t = (a_t - 1) / A (dt_t at A = 0)
 * in place of dt_t B_t u_t, so dt_t becomes c_t in gB and gu, the input term's derivative in gdt
 * is dc/ddt = a_t instead of 1 (gdt_t = sum_n lam_t a_t (h_{t-1} A + B_t u_t)), and gA gains
 * lam_t B_t u_t dc/dA (zoh_coef_dA); the adjoint recurrence is unchanged.
 * Each row keeps its forward states (fp64); the reductions over rows use per-thread fp64
 * partial sums added in thread order.
 * ---------------------------------------------------------------------------------------------- */

typedef struct {
    const orc_args* f;              /* forward inputs (y, last_state, rows unused) */
    const double *gy, *glast;
    double *gu, *gdelta, *gz;       /* (batch, D, L) */
    double *gh0;                    /* (batch, D, N) or NULL */
    /* per-thread partials: gB, gC (batch, N, L), gA (D, N), gD, gbias (D) */
    double *pB, *pC, *pA, *pD, *pbias;
    int64_t begin, end;
} orc_bwd_job;

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static void bwd_row(const orc_bwd_job* j, int64_t b, int64_t d, double* hist, double* lam) {
    const orc_args* a = j->f;
    const int64_t L = a->len, N = a->dstate, D = a->dim;
    const int64_t row_off = (b * D + d) * L;
    const int64_t bc_off = b * N * L;
    const double bias = a->delta_bias ? (double)a->delta_bias[d] : 0.0;
    const double dskip = a->Dvec ? (double)a->Dvec[d] : 0.0;
    /* forward, keeping h_{t} for t = -1 .. L-1 in hist[(t + 1) * N + n] */
    for (int64_t n = 0; n < N; ++n) hist[n] = a->h0 ? a->h0[(b * D + d) * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const double x = widen(a->delta, a->in_dtype, row_off + t) + bias;
        const double dt = a->delta_softplus ? softplus(x) : exp(x);
        const double ut = widen(a->u, a->in_dtype, row_off + t);
        for (int64_t n = 0; n < N; ++n) {
            const double Bt = widen(a->B, a->in_dtype, bc_off + n * L + t);
            const double An = (double)a->A[d * N + n];
            const double cf = a->zoh_b ? zoh_coef(dt, An) : dt;
            hist[(t + 1) * N + n] = exp(dt * An) * hist[t * N + n] + cf * Bt * ut;
        }
    }
    for (int64_t n = 0; n < N; ++n) lam[n] = j->glast ? j->glast[(b * D + d) * N + n] : 0.0;
    double gD = 0.0, gbias = 0.0;
    for (int64_t t = L - 1; t >= 0; --t) {
        const double x = widen(a->delta, a->in_dtype, row_off + t) + bias;
        const double dt = a->delta_softplus ? softplus(x) : exp(x);
        const double ut = widen(a->u, a->in_dtype, row_off + t);
        const double* h = hist + (t + 1) * N;
        const double* hprev = hist + t * N;
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) s += widen(a->C, a->in_dtype, bc_off + n * L + t) * h[n];
        const double p = s + dskip * ut;
        double g = 1.0;
        const double gyt = j->gy[row_off + t];
        if (a->z) {
            const double zt = widen(a->z, a->in_dtype, row_off + t);
            const double sg = sigmoid(zt);
            g = zt * sg;
            j->gz[row_off + t] = gyt * p * (sg + zt * sg * (1.0 - sg));
        }
        const double gp = gyt * g;
        gD += gp * ut;
        double gu = gp * dskip, gdt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double Bt = widen(a->B, a->in_dtype, bc_off + n * L + t);
            const double Ct = widen(a->C, a->in_dtype, bc_off + n * L + t);
            const double An = (double)a->A[d * N + n];
            const double an = exp(dt * An);
            const double cf = a->zoh_b ? zoh_coef(dt, An) : dt;    /* input coefficient */
            const double cf_dt = a->zoh_b ? an : 1.0;               /* its derivative in dt */
            lam[n] += gp * Ct;
            j->pC[bc_off + n * L + t] += gp * h[n];
            j->pB[bc_off + n * L + t] += lam[n] * cf * ut;
            gu += lam[n] * cf * Bt;
            gdt += lam[n] * (an * hprev[n] * An + cf_dt * Bt * ut);
            j->pA[d * N + n] += lam[n] * an * hprev[n] * dt;
            if (a->zoh_b) j->pA[d * N + n] += lam[n] * Bt * ut * zoh_coef_dA(dt, An);
            lam[n] *= an;
        }
        const double gx = a->delta_softplus ? gdt * sigmoid(x) : gdt * dt;
        j->gdelta[row_off + t] = gx;
        j->gu[row_off + t] = gu;
        gbias += gx;
    }
    if (j->gh0)
        for (int64_t n = 0; n < N; ++n) j->gh0[(b * D + d) * N + n] = lam[n];
    j->pD[d] += gD;
    j->pbias[d] += gbias;
}

static void* orc_bwd_worker(void* p) {
    const orc_bwd_job* j = (const orc_bwd_job*)p;
    const int64_t N = j->f->dstate;
    double* hist = (double*)malloc(sizeof(double) * (size_t)((j->f->len + 1) * N));
    double* lam = (double*)malloc(sizeof(double) * (size_t)N);
    if (!hist || !lam) {
        free(hist);
        free(lam);
        return (void*)1;
    }
    for (int64_t k = j->begin; k < j->end; ++k) bwd_row(j, k / j->f->dim, k % j->f->dim, hist, lam);
    free(hist);
    free(lam);
    return NULL;
}

/*
 * Gradients of the scan (all fp64, contiguous). gy (batch, D, L) is required; glast (batch, D, N)
 * may be NULL (no loss on the final state). Outputs: gu, gdelta (batch, D, L); gz (batch, D, L),
 * required when z is given; gB, gC (batch, N, L); gA (D, N); gD, gbias (D); gh0 (batch, D, N) or
 * NULL. gz/gD/gbias are written even when z/D/delta_bias are absent (then as if they were zero,
 * with gz left untouched). Returns 0, or a negative value on a bad argument or allocation failure.
 */
int oracle_selective_scan_bwd_ex(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int in_dtype,
                                 const void* u, const void* delta, const void* z, const void* B,
                                 const void* C, const float* A, const float* Dvec,
                                 const float* delta_bias, const double* h0, int delta_softplus,
                                 int zoh_b, const double* gy, const double* glast, double* gu,
                                 double* gdelta, double* gz, double* gB, double* gC, double* gA,
                                 double* gD, double* gbias, double* gh0, int nthreads) {
    if (batch <= 0 || dim <= 0 || len <= 0 || dstate <= 0) return -2;
    if (in_dtype != ORC_F32 && in_dtype != ORC_BF16) return -4;
    if (!u || !delta || !B || !C || !A || !gy || !gu || !gdelta || !gB || !gC || !gA || !gD || !gbias)
        return -1;
    if (z && !gz) return -1;
    orc_args f = {batch, dim, len, dstate, in_dtype, u, delta, z, B, C, A, Dvec, delta_bias, h0,
                  delta_softplus, zoh_b ? 1 : 0, NULL, batch * dim, NULL, NULL};
    const int64_t nrows = batch * dim;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > ORC_MAX_THREADS) nthreads = ORC_MAX_THREADS;
    if (nthreads > nrows) nthreads = (int)nrows;
    const int64_t nbc = batch * dstate * len, na = dim * dstate;
    const int64_t per_thread = 2 * nbc + na + 2 * dim;
    double* part = (double*)calloc((size_t)(per_thread * nthreads), sizeof(double));
    if (!part) return -8;
    orc_bwd_job jobs[ORC_MAX_THREADS];
    pthread_t tids[ORC_MAX_THREADS];
    const int64_t per = (nrows + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        double* q = part + per_thread * t;
        orc_bwd_job j = {&f, gy, glast, gu, gdelta, gz, gh0, q, q + nbc, q + 2 * nbc, q + 2 * nbc + na,
                         q + 2 * nbc + na + dim, per * t < nrows ? per * t : nrows,
                         per * (t + 1) < nrows ? per * (t + 1) : nrows};
        jobs[t] = j;
    }
    int ok = 1, started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, orc_bwd_worker, &jobs[t]) != 0) break;
        started = t;
    }
    if (orc_bwd_worker(&jobs[0]) != NULL) ok = 0;
    for (int t = 1; t <= started; ++t) {
        void* r = NULL;
        pthread_join(tids[t], &r);
        if (r != NULL) ok = 0;
    }
    for (int t = started + 1; t < nthreads; ++t)
        if (orc_bwd_worker(&jobs[t]) != NULL) ok = 0;
    if (ok) {
        for (int64_t i = 0; i < nbc; ++i) {
            double sb = 0.0, sc = 0.0;
            for (int t = 0; t < nthreads; ++t) {
                sb += jobs[t].pB[i];
                sc += jobs[t].pC[i];
            }
            gB[i] = sb;
            gC[i] = sc;
        }
        for (int64_t i = 0; i < na; ++i) {
            double s = 0.0;
            for (int t = 0; t < nthreads; ++t) s += jobs[t].pA[i];
            gA[i] = s;
        }
        for (int64_t i = 0; i < dim; ++i) {
            double sd = 0.0, sb = 0.0;
            for (int t = 0; t < nthreads; ++t) {
                sd += jobs[t].pD[i];
                sb += jobs[t].pbias[i];
            }
            gD[i] = sd;
            gbias[i] = sb;
        }
    }
    free(part);
    return ok ? 0 : -8;
}

/* The backward of the scan with Euler B. */
int oracle_selective_scan_bwd(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int in_dtype,
                              const void* u, const void* delta, const void* z, const void* B,
                              const void* C, const float* A, const float* Dvec,
                              const float* delta_bias, const double* h0, int delta_softplus,
                              const double* gy, const double* glast, double* gu, double* gdelta,
                              double* gz, double* gB, double* gC, double* gA, double* gD,
                              double* gbias, double* gh0, int nthreads) {
    return oracle_selective_scan_bwd_ex(batch, dim, len, dstate, in_dtype, u, delta, z, B, C, A, Dvec,
                                        delta_bias, h0, delta_softplus, 0, gy, glast, gu, gdelta, gz,
                                        gB, gC, gA, gD, gbias, gh0, nthreads);
}
