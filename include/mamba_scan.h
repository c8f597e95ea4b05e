/*
 * mamba_scan.h - C ABI of the MI355X (gfx950) selective-scan forward library.
 *
 * The operation (one call = the whole forward pass):
 *
 *   for every batch b, channel d, step t, state n (diagonal A):
 *     dt      = softplus(delta[b,d,t] + delta_bias[d])      if MAMBA_SCAN_DELTA_SOFTPLUS
 *             = exp(delta[b,d,t] + delta_bias[d])           otherwise
 *     h[n]    = exp(dt * A[d,n]) * h[n] + dt * B[b,n,t] * u[b,d,t]      (h starts at h0 or 0)
 *     y[b,d,t]= (sum_n C[b,n,t] * h[n] + D[d] * u[b,d,t]) * silu(z[b,d,t])
 *   last_state[b,d,n] = h[n] after the last step.
 *
 * Sources: "Mamba代码实战：手把手教你用PyTorch复现选择性扫描核心逻辑（附避坑指南）" - §2.1 (tensor
 * layouts), §2.2 and §6 (delta + delta_bias, then softplus or exp; the argument list
 * u, delta, A, B, C, D, delta_bias, delta_softplus, return_last_state; the returned state),
 * §3.1 (dA = exp(delta*A), dB = delta*B), §3.2 (the per-step recurrence from a zero state),
 * §3.3 (skip y + u*D, then the gate y * silu(z)), §4.1 (unit stride along L);
 * "Mamba-minimal项目解析：深入理解Mamba模型的极简实现", 关键技术点 1 (y = sum_n h[n] * C[n]) and 5
 * (A = -exp(A_log) and D in fp32, softplus on delta); "手把手用PyTorch实现Mamba的SSM层从HiPPO矩阵到
 * 选择性扫描算法" §3.1 (a scan that starts from a given state: the optional h0).
 *
 * Conventions
 *  - All pointers are DEVICE pointers (memory of the GPU that is current when the call is made).
 *    The caller owns every buffer; the library never allocates, frees or synchronises.
 *  - u, delta, z: (batch, dim, len); B, C: (batch, dstate, len); all in `dtype`.
 *    A: (dim, dstate), D: (dim), delta_bias: (dim), h0: (batch, dim, dstate): fp32.
 *    y: (batch, dim, len) fp32; last_state: (batch, dim, dstate) fp32.
 *  - Strides are in elements. The innermost stride (len for u/delta/z/B/C/y, dstate for
 *    A/h0/last_state) must be 1; the other strides are free (slices are fine) but must be >= 0.
 *    A NULL strides argument means every tensor is contiguous.
 *  - z, D, delta_bias, h0 may be NULL (absent: no gate, no skip, no bias, zero initial state).
 *    last_state must be non-NULL exactly when MAMBA_SCAN_RETURN_LAST_STATE is set (it may be
 *    NULL in an empty call, below).
 *  - Empty calls (ABI 13): batch, dim and len may be 0 (dstate must be at least 1). A tensor with
 *    no elements is never read or written and its pointer may be NULL. With batch * dim = 0 the
 *    call enqueues nothing. With len = 0, y has no elements and last_state, when requested,
 *    receives h0, or zeros without h0: a scan of no steps leaves its initial state (one launch
 *    of the generic kernel). A forced kernel is not used in an empty call.
 *  - Outputs must not overlap any input or each other.
 *  - The work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 *    returns without waiting. Calls on different streams may run concurrently.
 *  - Errors are returned before anything is enqueued (codes below); the library never aborts.
 *    mamba_scan_strerror() turns a code into a message.
 *  - Thread-safe: no mutable global state.
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA_SCAN_ABI_VERSION 15

/* Storage dtype of u, delta, z, B, C. Arithmetic is fp32 in every case. */
typedef enum mamba_scan_dtype {
    MAMBA_SCAN_F32 = 0,
    MAMBA_SCAN_BF16 = 1
} mamba_scan_dtype;

/* flags */
#define MAMBA_SCAN_DELTA_SOFTPLUS (1u << 0)    /* dt = softplus(.) ; clear: dt = exp(.) */
#define MAMBA_SCAN_RETURN_LAST_STATE (1u << 1) /* write last_state */
/* B discretised by zero-order hold: the input term becomes (exp(dt*A[d,n]) - 1) / A[d,n] * B * u
 * (dt * B * u where A[d,n] = 0) instead of dt * B * u. "手把手用PyTorch实现Mamba的SSM层…" §2.1:
 * B_d = A^-1 (e^{A dt} - I) B, for a diagonal A. Run by the lane-per-state kernels at dstate 16,
 * 32 and 64 (ABI 9), the chunked kernel (ABI 11) and the short-call kernel (ABI 12), else by the
 * tiled or generic one. The backward pass takes it from ABI 14 (see mamba_scan_bwd). */
#define MAMBA_SCAN_ZOH_B (1u << 2)
/* Save the state before every 16-step segment, for the backward pass: the forward writes
 * h before steps 0, 16, 32, ... of every (b, d) row to the workspace, laid out (batch, dim,
 * ceil(len/16), dstate) fp32 contiguous (mamba_scan_workspace_bytes gives its size with this
 * flag), and mamba_scan_bwd, given them as `checkpoints`, skips recomputing them. The
 * lane-per-state kernels (dstate 16, 32 or 64) and, from ABI 10, the chunked kernel (dstate 16:
 * the default where it is the default without the flag; its states come from its combine, so they
 * agree with the sequential recurrence's to rounding; not with ZOH_B); with ZOH_B the
 * lane-per-state kernels (ABI 15); MAMBA_SCAN_ERR_UNSUPPORTED otherwise. ABI version 6. */
#define MAMBA_SCAN_SAVE_CHECKPOINTS (1u << 3)
/* Kernel selection, for testing and tuning; at most one of these bits (MAMBA_SCAN_ERR_ARGS
 * otherwise). Default (none): with 16 states, the short-call kernel for at most 4 steps and the
 * chunked kernel for at least 1024 steps when too few (batch, channel) rows would give every SIMD
 * of the GPU two waves of the lane-per-state kernel; otherwise the lane-per-state kernel where it
 * can run, else the tiled one, else the generic one. The backward pass takes FORCE_TILED and
 * FORCE_LANES too (ABI 8; see mamba_scan_bwd). */
#define MAMBA_SCAN_FORCE_GENERIC (1u << 8) /* one lane per row, any shape and alignment */
#define MAMBA_SCAN_FORCE_TILED (1u << 9)   /* the LDS-tiled kernel; error if it cannot run */
#define MAMBA_SCAN_FORCE_LANES (1u << 10)  /* one 16-lane row per channel, one lane per state
                                              at dstate 16 and dstate/16 states per lane at 32
                                              or 64; ZOH_B from ABI 9; error if it cannot run
                                              (ABI 5) */
/* Chunked along the sequence (ABI 7): one wave per channel, its four 16-lane rows scan four
 * consecutive 16-step runs of each 64-step chunk and are combined with the associative (a, b)
 * operator of the parallel scan ("手把手用PyTorch实现Mamba的SSM层…" §3.2), the state carried
 * from chunk to chunk in registers. dstate 16; SAVE_CHECKPOINTS from ABI 10, ZOH_B from ABI 11,
 * not both; error if it cannot run. Results agree with the sequential kernels to rounding (not bit for bit); a sequence split
 * at a multiple of 64 steps and resumed from last_state gives the same bits as one call. */
#define MAMBA_SCAN_FORCE_CHUNKED (1u << 11)
/* Short calls (ABI 7): one lane per (channel, state), each step in registers with no LDS staging
 * and no barrier; for recurrent decode (one or a few steps per call from the previous call's
 * last_state, "告别'炼丹'…" §2.1 times single-step inference). dstate 16 (ZOH_B from ABI 12), no
 * SAVE_CHECKPOINTS, at most 64 steps; the default for calls of at most 4 steps. Its states are the
 * same bits as the lane-per-state kernel's, with either input term; y may differ in the last bits (the 16 states' terms
 * are added in another order). */
#define MAMBA_SCAN_FORCE_STEP (1u << 12)
#define MAMBA_SCAN_KNOWN_FLAGS 0x1F0Fu

/* error codes */
#define MAMBA_SCAN_OK 0
#define MAMBA_SCAN_ERR_NULL (-1)      /* a required pointer is NULL */
#define MAMBA_SCAN_ERR_SHAPE (-2)     /* a dimension < 0, dstate < 1, or a stride < 0 */
#define MAMBA_SCAN_ERR_STRIDE (-3)    /* an innermost stride is not 1 */
#define MAMBA_SCAN_ERR_DTYPE (-4)     /* unknown dtype */
#define MAMBA_SCAN_ERR_DSTATE (-5)    /* dstate above MAMBA_SCAN_MAX_DSTATE */
#define MAMBA_SCAN_ERR_ARGS (-6)      /* flags/pointer mismatch, unknown flag, overlapping buffers */
#define MAMBA_SCAN_ERR_LAUNCH (-7)    /* the HIP runtime refused the launch */
#define MAMBA_SCAN_ERR_UNSUPPORTED (-8) /* a forced kernel, or SAVE_CHECKPOINTS, cannot run
                                           this shape/alignment */
#define MAMBA_SCAN_ERR_WORKSPACE (-9) /* workspace too small for the requested plan */
#define MAMBA_SCAN_ERR_SCRATCH (-10)  /* mamba_scan_bwd_static: the call needs more workspace than
                                         MAMBA_SCAN_STATIC_SCRATCH_BYTES */

#define MAMBA_SCAN_MAX_DSTATE 256

typedef struct mamba_scan_ptrs {
    const void* u;           /* (batch, dim, len) dtype, required */
    const void* delta;       /* (batch, dim, len) dtype, required */
    const void* z;           /* (batch, dim, len) dtype, or NULL */
    const void* B;           /* (batch, dstate, len) dtype, required */
    const void* C;           /* (batch, dstate, len) dtype, required */
    const float* A;          /* (dim, dstate) fp32, required */
    const float* D;          /* (dim) fp32, or NULL */
    const float* delta_bias; /* (dim) fp32, or NULL */
    const float* h0;         /* (batch, dim, dstate) fp32, or NULL (zero initial state) */
    float* y;                /* (batch, dim, len) fp32, required, written */
    float* last_state;       /* (batch, dim, dstate) fp32, written iff RETURN_LAST_STATE */
    void* workspace;         /* the saved states with MAMBA_SCAN_SAVE_CHECKPOINTS, else unused
                                (may be NULL); see mamba_scan_workspace_bytes */
    int64_t workspace_bytes; /* its size in bytes */
} mamba_scan_ptrs;

typedef struct mamba_scan_shape {
    int64_t batch, dim, len, dstate;
} mamba_scan_shape;

/* Element strides: [0] batch, [1] dim or state, [2] len (must be 1) for the 3-d tensors;
 * A: [0] dim, [1] state (must be 1); D, delta_bias: stride along dim. */
typedef struct mamba_scan_strides {
    int64_t u[3], delta[3], z[3];
    int64_t B[3], C[3];
    int64_t y[3];
    int64_t h0[3], last_state[3];
    int64_t A[2];
    int64_t D, delta_bias;
} mamba_scan_strides;

/* Enqueue the selective-scan forward pass on `stream`. Returns MAMBA_SCAN_OK or an error code. */
int mamba_scan_fwd(const mamba_scan_ptrs* p, const mamba_scan_shape* s,
                   const mamba_scan_strides* st, mamba_scan_dtype dtype, uint32_t flags,
                   void* stream);

/* The kernel mamba_scan_fwd would run for these arguments (ABI 7): one of the values below, or
 * the error code mamba_scan_fwd would return before launching. Enqueues nothing; the pointers are
 * only compared (overlaps, alignment), never dereferenced. The choice between the chunked and
 * the lane-per-state kernel depends on the current device's compute-unit count. An empty call
 * gives MAMBA_SCAN_KERNEL_NONE when it enqueues nothing and MAMBA_SCAN_KERNEL_GENERIC when it
 * writes last_state (ABI 13). */
#define MAMBA_SCAN_KERNEL_NONE 0
#define MAMBA_SCAN_KERNEL_GENERIC 1
#define MAMBA_SCAN_KERNEL_TILED 2
#define MAMBA_SCAN_KERNEL_LANES 3
#define MAMBA_SCAN_KERNEL_CHUNKED 4
#define MAMBA_SCAN_KERNEL_STEP 5
int mamba_scan_fwd_kernel(const mamba_scan_ptrs* p, const mamba_scan_shape* s,
                          const mamba_scan_strides* st, mamba_scan_dtype dtype, uint32_t flags);

/* Bytes of device workspace mamba_scan_fwd needs with these flags: 0 without
 * MAMBA_SCAN_SAVE_CHECKPOINTS (no forward kernel uses scratch memory: the chunked kernel carries
 * the state between chunks of the sequence in registers); with it, the size of the saved states,
 * which the call then requires (MAMBA_SCAN_ERR_WORKSPACE below it; 4-byte alignment,
 * MAMBA_SCAN_ERR_ARGS otherwise). Negative on invalid arguments. */
int64_t mamba_scan_workspace_bytes(const mamba_scan_shape* s, mamba_scan_dtype dtype,
                                   uint32_t flags);

/*
 * Backward pass (ABI version 2; any dstate from version 4).
 *
 * Gradients of a scalar loss that depends on the forward pass above through y (gradient dy)
 * and, optionally, through last_state (gradient dlast_state). Sources: "手把手用PyTorch实现Mamba的
 * SSM层…" §4.2 (memory-efficient training: the states are recomputed for the backward pass, not
 * stored by the forward pass) and "Mamba代码实战…" §7 (item 3, an efficient backward pass); the
 * function differentiated is the forward operation defined at the top of this file. With
 * x = delta + delta_bias, dt = softplus(x) or exp(x), a = exp(dt*A), p = sum_n C*h + D*u:
 *   dz = dy * p * silu'(z);   dD[d] = sum_{b,t} dy*silu(z)*u;   dh0 = dLoss/d(initial state)
 *   du, ddelta (= dLoss/dx), dB, dC, dA, ddelta_bias[d] = sum_{b,t} ddelta
 * by the chain rule through the recurrence, in reverse step order.
 *
 * Conventions
 *  - Every tensor is CONTIGUOUS in the layouts of the forward pass (no strides argument).
 *  - Forward inputs as in mamba_scan_ptrs (u, delta, z, B, C in `dtype`; A, D, delta_bias, h0
 *    fp32; z, D, delta_bias, h0 may be NULL). The forward's output is not needed.
 *  - dy (batch, dim, len) fp32 is required; dlast_state (batch, dim, dstate) fp32 may be NULL
 *    (no loss on the final state).
 *  - Gradients, all fp32, all written in full (never accumulated into): du, ddelta
 *    (batch, dim, len), required; dz (batch, dim, len), required exactly when z is given;
 *    dB, dC (batch, dstate, len), required; dA (dim, dstate), required; dD and ddelta_bias (dim),
 *    each required exactly when D / delta_bias is given; dh0 (batch, dim, dstate) or NULL.
 *  - Workspace: mamba_scan_bwd_workspace_bytes() bytes or more (queried with the call's flags,
 *    plus MAMBA_SCAN_SAVE_CHECKPOINTS when `checkpoints` is given), 256-byte aligned, device
 *    memory owned by the caller (states every 16 steps unless given; partial sums of dB and dC
 *    per group of channels, 16 channels for the lane-per-state kernel, 64 for the segment-tiled
 *    one, which also keeps fp32 copies of B and C; for few long rows the lane-per-state kernel
 *    splits the sequence into parts run side by side and keeps per-part partial sums of dA, dD,
 *    dbias and the adjoint handed from part to part).
 *  - Flags: MAMBA_SCAN_DELTA_SOFTPLUS, MAMBA_SCAN_ZOH_B (ABI 14: the gradients of the forward
 *    with zero-order-hold B, where the input term's coefficient c = (exp(dt*A) - 1) / A replaces
 *    dt in dB and du, its derivative exp(dt*A) enters ddelta, and dA gains
 *    sum lam*B*u*dc/dA; the segment-tiled kernel from ABI 14, the lane-per-state one and
 *    `checkpoints` saved by a zero-order-hold forward from ABI 15), and at most one of the
 *    kernel choices (ABI 8; MAMBA_SCAN_ERR_ARGS for both or any other flag):
 *      MAMBA_SCAN_FORCE_LANES: the lane-per-state backward, one lane per (channel, state) as in
 *        the forward lane-per-state kernel, 16-step segments walked in reverse from the states
 *        saved every 16 steps (given, or written first by the forward launch that a call with
 *        MAMBA_SCAN_SAVE_CHECKPOINTS would make, its y going to du); dstate 16, 32 or 64 and
 *        row byte offsets within 31 bits
 *        (MAMBA_SCAN_ERR_UNSUPPORTED otherwise). The default wherever it can run.
 *      MAMBA_SCAN_FORCE_TILED: the segment-tiled backward (64 channels per workgroup, at most 2
 *        states per wave), any dstate.
 *    The two give the same gradients to rounding, not bit for bit; each is deterministic.
 *  - Empty calls (ABI 13): batch, dim and len may be 0, as in the forward (tensors with no
 *    elements are never touched and may be NULL). No scan runs and the workspace may be empty
 *    (mamba_scan_bwd_workspace_bytes gives 0); the gradients that have elements are sums over
 *    nothing and are written as zeros (dA, dD, ddelta_bias; dB and dC when dim = 0), except dh0,
 *    which with len = 0 receives dlast_state (or zeros without it): the initial state of a scan
 *    of no steps is its final state.
 *  - Any dstate up to MAMBA_SCAN_MAX_DSTATE. Above 16 the states are processed in blocks of at
 *    most 16, one launch each (either kernel): du, ddelta and dz are accumulated in place across
 *    the blocks, in block order, so their values can differ in the last bits from a one-block
 *    sum.
 *  - checkpoints (ABI 6): NULL, or the states that a forward call with
 *    MAMBA_SCAN_SAVE_CHECKPOINTS saved for the same inputs (same h0 included), 4-byte aligned;
 *    the scan then starts from them instead of recomputing them. The caller guarantees that they
 *    belong to these inputs: nothing checks it.
 *  - Outputs may not overlap each other, any input or the workspace (MAMBA_SCAN_ERR_ARGS).
 *  - Enqueued on `stream`: lane-per-state, the forward that writes the states (unless given),
 *    the backward scan (one launch per block of 16 states), a fixed-order reduction; segment-tiled, B/C widening, the scan (one
 *    launch per block of states), the same reduction. Results are bitwise deterministic.
 */
typedef struct mamba_scan_bwd_ptrs {
    const void* u;                /* forward inputs */
    const void* delta;
    const void* z;
    const void* B;
    const void* C;
    const float* A;
    const float* D;
    const float* delta_bias;
    const float* h0;
    const float* dy;              /* (batch, dim, len) fp32, required */
    const float* dlast_state;     /* (batch, dim, dstate) fp32, or NULL */
    float* du;                    /* (batch, dim, len) */
    float* ddelta;                /* (batch, dim, len) */
    float* dz;                    /* (batch, dim, len) iff z */
    float* dB;                    /* (batch, dstate, len) */
    float* dC;                    /* (batch, dstate, len) */
    float* dA;                    /* (dim, dstate) */
    float* dD;                    /* (dim) iff D */
    float* ddelta_bias;           /* (dim) iff delta_bias */
    float* dh0;                   /* (batch, dim, dstate) or NULL */
    void* workspace;
    int64_t workspace_bytes;
    const float* checkpoints;     /* (batch, dim, ceil(len/16), dstate) fp32 states saved by the
                                     forward (MAMBA_SCAN_SAVE_CHECKPOINTS) on the same inputs, or
                                     NULL: recomputed (ABI version 6) */
} mamba_scan_bwd_ptrs;

int mamba_scan_bwd(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape* s, mamba_scan_dtype dtype,
                   uint32_t flags, void* stream);

/*
 * Backward pass that allocates nothing (ABI 7), for callers that cannot allocate device memory:
 * code under HIP graph capture, tight training or serving loops, harnesses that forbid
 * allocation. The same operation, arguments and results as mamba_scan_bwd (bit for bit), except
 * that the workspace is the library's own static buffer of MAMBA_SCAN_STATIC_SCRATCH_BYTES on each
 * device: p->workspace must be NULL and p->workspace_bytes 0 (MAMBA_SCAN_ERR_ARGS otherwise). A
 * call whose workspace (mamba_scan_bwd_workspace_bytes, queried with MAMBA_SCAN_SAVE_CHECKPOINTS
 * when checkpoints are given) exceeds it returns MAMBA_SCAN_ERR_SCRATCH before enqueuing anything.
 * No call allocates or frees memory; the first call on a device looks up that device's buffer.
 *  - The buffer of a GPU is held from the library's first use on it until the process ends.
 *  - Every call on one GPU uses that GPU's buffer: calls that overlap in time on the same GPU
 *    (on different streams, or from different host threads) race and must not be made; calls
 *    one after another on a stream are fine. The buffer keeps the last call's contents; the
 *    backward writes every part of it that it reads, so nothing has to be cleared.
 * At the Mamba-130m layer (batch 8, dim 1536, dstate 16, len 2048) the segment-tiled kernel
 * (MAMBA_SCAN_FORCE_TILED) from the forward's saved states needs 53 MB and fits; the lane-per-state
 * kernel needs 201 MB there (its dB / dC partial sums) and recomputing the states 154 MB
 * (segment-tiled) or 302 MB: those are refused.
 */
#define MAMBA_SCAN_STATIC_SCRATCH_BYTES (64ll << 20)
int mamba_scan_bwd_static(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape* s, mamba_scan_dtype dtype,
                          uint32_t flags, void* stream);

/* Workspace bytes mamba_scan_bwd needs for this shape (> 0), or a negative error code. Flags:
 * MAMBA_SCAN_DELTA_SOFTPLUS (ignored for the size), the call's kernel choice (FORCE_LANES or
 * FORCE_TILED, ABI 8; none: the default kernel's size; MAMBA_SCAN_ERR_UNSUPPORTED where the
 * forced kernel cannot run) and MAMBA_SCAN_SAVE_CHECKPOINTS, meaning that the call will be given
 * `checkpoints`: the size then leaves out the recomputed states (ABI 7). */
int64_t mamba_scan_bwd_workspace_bytes(const mamba_scan_shape* s, mamba_scan_dtype dtype, uint32_t flags);

/*
 * Upstream stages of a Mamba block (ABI version 3): the producer of the scan's inputs.
 *
 *   u[b,d,t]     = bf16( silu( conv_b[d] + sum_k conv_w[d,k] * x[b,d,t-(d_conv-1)+k] ) )
 *                  (x = 0 before t = 0: a causal depthwise convolution)
 *   xdbl[b,j,t]  = bf16( sum_d w_x[j,d] * u[b,d,t] )              j < dt_rank + 2*dstate
 *   delta[b,d,t] = bf16( sum_{r < dt_rank} w_dt[d,r] * xdbl[b,r,t] )
 * bf16() rounds fp32 to the nearest bf16 (ties to even); the sums are accumulated in fp32.
 * The scan's B and C are then rows dt_rank .. dt_rank+dstate-1 and dt_rank+dstate .. of xdbl
 * (batch stride (dt_rank + 2*dstate)*len, state stride len), and dt_proj's bias is the scan's
 * delta_bias (the scan adds it before its softplus).
 *
 * Sources: "告别'炼丹'：从Mamba-minimal入手，亲手调参并可视化SSM的状态变化" §1.1 (MambaBlock: Conv1d
 * with kernel d_conv and padding d_conv-1, x_proj = Linear(d_inner, dt_rank + 2*d_state),
 * dt_proj = Linear(dt_rank, d_inner)) and §2.2 (the dt rows are x_dbl[..., :dt_rank]);
 * "Mamba-minimal项目解析：深入理解Mamba模型的极简实现" §4 (x_proj without bias, dt_proj with bias)
 * and §5 (x_dbl splits into delta, B, C in that order; softplus(dt_proj(delta))). The convolution
 * is read as depthwise (groups = channels, as the conv-gated block of "手把手用PyTorch实现Mamba的SSM层…"
 * §5.2 builds it) and causal (the first len outputs of the padded convolution), followed by SiLU.
 *
 * Conventions
 *  - Device pointers; every tensor CONTIGUOUS: x, u, delta (batch, dim, len) bf16; xdbl
 *    (batch, dt_rank + 2*dstate, len) bf16; conv_w (dim, d_conv) fp32; conv_b (dim) fp32 or NULL
 *    (no bias); w_x (dt_rank + 2*dstate, dim) bf16; w_dt (dim, dt_rank) bf16 (row-major, as the
 *    weights of the layers above).
 *  - dtype must be MAMBA_SCAN_BF16 (MAMBA_SCAN_ERR_UNSUPPORTED for MAMBA_SCAN_F32,
 *    MAMBA_SCAN_ERR_DTYPE for an unknown value).
 *  - Supported (MAMBA_SCAN_ERR_UNSUPPORTED otherwise): len % 4 == 0, dim % 8 == 0 and
 *    dim <= 4096, dt_rank % 8 == 0 and dt_rank <= 64, dt_rank + 2*dstate <= 128,
 *    1 <= d_conv <= 4, dim*len and (dt_rank + 2*dstate)*len below 2^30 (one batch of a tensor
 *    under 2 GiB); x, u, delta, xdbl 8-byte aligned; w_x, w_dt 16-byte aligned.
 *  - u, xdbl and delta are written in full; they may not overlap each other or any input
 *    (MAMBA_SCAN_ERR_ARGS).
 *  - Enqueued on `stream` as one kernel; results are bitwise deterministic.
 */
typedef struct mamba_upstream_ptrs {
    const void* x;        /* (batch, dim, len) bf16 */
    const float* conv_w;  /* (dim, d_conv) */
    const float* conv_b;  /* (dim) or NULL */
    const void* w_x;      /* (dt_rank + 2*dstate, dim) bf16 */
    const void* w_dt;     /* (dim, dt_rank) bf16 */
    void* u;              /* out: (batch, dim, len) bf16 */
    void* xdbl;           /* out: (batch, dt_rank + 2*dstate, len) bf16 */
    void* delta;          /* out: (batch, dim, len) bf16 */
} mamba_upstream_ptrs;

typedef struct mamba_upstream_shape {
    int64_t batch, dim, len, dstate, dt_rank, d_conv;
} mamba_upstream_shape;

int mamba_block_upstream(const mamba_upstream_ptrs* p, const mamba_upstream_shape* s,
                         mamba_scan_dtype dtype, void* stream);

/* Static message for an error code; never NULL. */
const char* mamba_scan_strerror(int code);

/* MAMBA_SCAN_ABI_VERSION of the built library. */
int mamba_scan_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
