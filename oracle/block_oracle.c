/*
 * fp64 CPU oracle of the part of a Mamba block that feeds the selective scan: the causal
 * depthwise convolution with SiLU, the x projection and the dt projection.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file:
 * only the tests, the smoke check and the bench's CPU-baseline leg use it. It shares no code,
 * header, table or helper with the HIP library.
 *
 * What it computes, in the order of the pages:
 *   - "告别'炼丹'：从Mamba-minimal入手，亲手调参并可视化SSM的状态变化" §1.1 (the MambaBlock listing):
 *       conv1d = Conv1d(d_inner, d_inner, kernel d_conv, padding d_conv - 1);
 *       x_proj = Linear(d_inner, dt_rank + 2 d_state);  dt_proj = Linear(dt_rank, d_inner);
 *     §2.2 the dt rows are x_dbl[..., :dt_rank] and delta = softplus(dt_proj(those rows)).
 *   - "Mamba-minimal项目解析：深入理解Mamba模型的极简实现" §4 (x_proj has no bias, dt_proj has one)
 *     and §5 (x_dbl is split into delta, B, C in that order; delta = softplus(dt_proj(delta))).
 * Readings where the pages leave a step open:
 *   - the convolution is depthwise (one 1-D filter per channel), as the conv-gated SSM block of
 *     "手把手用PyTorch实现Mamba的SSM层…" §5.2 builds it (groups = channels), and causal: with
 *     padding d_conv - 1 the first L outputs are kept, so output t sees inputs t-d_conv+1 .. t;
 *   - SiLU follows the convolution (the block's forward is not printed; SiLU is the activation
 *     the pages use in the block, on the gate);
 *   - dt_proj's bias is not added here: it is the scan's delta_bias, which the scan adds before
 *     its softplus, so softplus(dt_proj(x)) is computed exactly once, inside the scan;
 *   - storage precision is the model dtype bf16 (the mixed-precision advice of the same page,
 *     §6.1, and of the Mamba-minimal page's optimisation list): the convolution output u, the
 *     projection x_dbl and delta are each rounded once to bf16 (round to nearest, ties to even),
 *     and the next stage reads the rounded values.
 * Arithmetic between the rounding points is fp64. PyTorch's Conv1d is a cross-correlation:
 *   out[d, t] = bias[d] + sum_k w[d, k] * xpad[d, t + k],  xpad = x with d_conv - 1 zeros in front.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, 4);
    return (double)f;
}

/* v rounded to the nearest bf16 value (8 significant bits, ties to even), as its bit pattern.
 * |v| = m 2^e with m in [0.5, 1): the bf16 spacing there is 2^(e-8), and 2^-133 below 2^-126. */
static uint16_t round_bf16(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    int e;
    frexp(fabs(v), &e);
    int q = e - 8;
    if (q < -133) q = -133;
    const double w = ldexp(nearbyint(ldexp(v, -q)), q); /* default rounding mode: ties to even */
    const float f = (float)w;                             /* exact: w has at most 8 bits */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return (uint16_t)(bits >> 16);
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

typedef struct {
    int64_t batch, dim, len, dstate, dt_rank, d_conv;
    const uint16_t* x;
    const float *conv_w, *conv_b;
    const uint16_t *w_x, *w_dt;
    uint16_t *u, *xdbl, *delta;
    double *u_pre, *xdbl_pre, *delta_pre;
} up_args;

/* Stage 1, one (b, d) row: u = bf16(silu(conv)). */
static void conv_row(const up_args* a, int64_t b, int64_t d, double* scratch) {
    (void)scratch;
    const int64_t L = a->len, K = a->d_conv, off = (b * a->dim + d) * L;
    for (int64_t t = 0; t < L; ++t) {
        double acc = a->conv_b ? (double)a->conv_b[d] : 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t s = t + k - (K - 1); /* xpad[t + k] */
            if (s >= 0) acc += (double)a->conv_w[d * K + k] * bf16_value(a->x[off + s]);
        }
        const double v = silu(acc);
        if (a->u_pre) a->u_pre[off + t] = v;
        a->u[off + t] = round_bf16(v);
    }
}

/* Stage 2, one (b, j) row: x_dbl[b, j, :] = sum_d w_x[j, d] u[b, d, :], rounded to bf16. */
static void xproj_row(const up_args* a, int64_t b, int64_t j, double* acc) {
    const int64_t L = a->len, D = a->dim, J = a->dt_rank + 2 * a->dstate;
    for (int64_t t = 0; t < L; ++t) acc[t] = 0.0;
    for (int64_t d = 0; d < D; ++d) {
        const double w = bf16_value(a->w_x[j * D + d]);
        const uint16_t* ur = a->u + (b * D + d) * L;
        for (int64_t t = 0; t < L; ++t) acc[t] += w * bf16_value(ur[t]);
    }
    const int64_t off = (b * J + j) * L;
    for (int64_t t = 0; t < L; ++t) {
        if (a->xdbl_pre) a->xdbl_pre[off + t] = acc[t];
        a->xdbl[off + t] = round_bf16(acc[t]);
    }
}

/* Stage 3, one (b, d) row: delta[b, d, :] = sum_r w_dt[d, r] x_dbl[b, r, :] over the first
 * dt_rank rows of x_dbl, rounded to bf16. */
static void dtproj_row(const up_args* a, int64_t b, int64_t d, double* acc) {
    const int64_t L = a->len, R = a->dt_rank, J = a->dt_rank + 2 * a->dstate;
    for (int64_t t = 0; t < L; ++t) acc[t] = 0.0;
    for (int64_t r = 0; r < R; ++r) {
        const double w = bf16_value(a->w_dt[d * R + r]);
        const uint16_t* xr = a->xdbl + (b * J + r) * L;
        for (int64_t t = 0; t < L; ++t) acc[t] += w * bf16_value(xr[t]);
    }
    const int64_t off = (b * a->dim + d) * L;
    for (int64_t t = 0; t < L; ++t) {
        if (a->delta_pre) a->delta_pre[off + t] = acc[t];
        a->delta[off + t] = round_bf16(acc[t]);
    }
}

typedef void (*row_fn)(const up_args*, int64_t, int64_t, double*);

typedef struct {
    const up_args* a;
    row_fn fn;
    int64_t rows_per_batch, nitems, first, stride;
    int failed;
} up_job;

static void* up_worker(void* p) {
    up_job* j = (up_job*)p;
    double* acc = (double*)malloc(sizeof(double) * (size_t)j->a->len);
    if (!acc) {
        j->failed = 1;
        return NULL;
    }
    for (int64_t k = j->first; k < j->nitems; k += j->stride)
        j->fn(j->a, k / j->rows_per_batch, k % j->rows_per_batch, acc);
    free(acc);
    return NULL;
}

#define UP_MAX_THREADS 256

/* Items k = b * rows_per_batch + r, thread i takes k = i, i + nthreads, ... */
static int run_stage(const up_args* a, row_fn fn, int64_t rows_per_batch, int nthreads) {
    const int64_t nitems = a->batch * rows_per_batch;
    if (nthreads > nitems) nthreads = (int)nitems;
    pthread_t th[UP_MAX_THREADS];
    up_job jobs[UP_MAX_THREADS];
    int started = 0, failed = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (up_job){a, fn, rows_per_batch, nitems, i, nthreads, 0};
        if (nthreads == 1) {
            up_worker(&jobs[i]);
        } else if (pthread_create(&th[i], NULL, up_worker, &jobs[i]) == 0) {
            ++started;
        } else {
            jobs[i].failed = 1;
        }
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i) failed |= jobs[i].failed;
    return failed ? -10 : 0;
}

/*
 * x (batch, dim, len) bf16 bits; conv_w (dim, d_conv) fp32; conv_b (dim) fp32 or NULL;
 * w_x (dt_rank + 2 dstate, dim) bf16 bits; w_dt (dim, dt_rank) bf16 bits; all contiguous.
 * Writes u (batch, dim, len), xdbl (batch, dt_rank + 2 dstate, len), delta (batch, dim, len) as
 * bf16 bits, and when non-NULL the fp64 values before each rounding (u_pre, xdbl_pre, delta_pre,
 * same shapes). Returns 0, or a negative value on a bad argument or a failed thread.
 */
int oracle_block_upstream(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int64_t dt_rank,
                          int64_t d_conv, const uint16_t* x, const float* conv_w,
                          const float* conv_b, const uint16_t* w_x, const uint16_t* w_dt,
                          uint16_t* u, uint16_t* xdbl, uint16_t* delta, double* u_pre,
                          double* xdbl_pre, double* delta_pre, int nthreads) {
    if (batch <= 0 || dim <= 0 || len <= 0 || dstate <= 0 || dt_rank <= 0 || d_conv <= 0) return -2;
    if (!x || !conv_w || !w_x || !w_dt || !u || !xdbl || !delta) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > UP_MAX_THREADS) nthreads = UP_MAX_THREADS;
    const up_args a = {batch, dim, len, dstate, dt_rank, d_conv, x, conv_w, conv_b, w_x, w_dt,
                       u, xdbl, delta, u_pre, xdbl_pre, delta_pre};
    int rc = run_stage(&a, conv_row, dim, nthreads);
    if (rc == 0) rc = run_stage(&a, xproj_row, dt_rank + 2 * dstate, nthreads);
    if (rc == 0) rc = run_stage(&a, dtproj_row, dim, nthreads);
    return rc;
}

/* The rounding above, exposed so that tests can pin it against other implementations. */
void oracle_round_bf16(const double* v, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(v[i]);
}
