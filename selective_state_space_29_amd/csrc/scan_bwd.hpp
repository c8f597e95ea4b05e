// Backward pass of the selective scan for gfx950: the gradients of a loss that reaches the scan
// through y (dy) and, optionally, through the final state (dlast_state).
//
// What is differentiated is the forward recurrence of "Mamba代码实战…" §3.1-§3.3 and §6 (with the
// output contraction of "Mamba-minimal项目解析…" 关键技术点 1 and the optional initial state of
// "手把手用PyTorch实现Mamba的SSM层…" §3.1). As "手把手用PyTorch实现Mamba的SSM层…" §4.2 (memory-efficient
// training) prescribes, no per-step state is stored: the states are recomputed. With
// x = delta + bias, dt = softplus(x) (or exp(x)), a = exp(dt A), h_t = a h_{t-1} + dt B_t u_t,
// p_t = sum_n C_t h_t + D u_t, y_t = p_t g_t (g = silu(z), or 1), and lam = dLoss/dh:
//   gp = dy g;  lam_t += gp C_t;  dC += gp h_t;  dB += lam dt u;  du = gp D + dt sum_n lam B
//   ddt = sum_n lam (a h_{t-1} A + B u);  dA += lam a h_{t-1} dt;  ddelta = ddt softplus'(x)
//   dz = dy p silu'(z);  dD += gp u;  dbias += ddelta;  then lam_{t-1} = a lam_t;  dh0 = lam.
// With B discretised by zero-order hold ("手把手用PyTorch实现Mamba的SSM层…" §2.1, diagonal A) the
// input term is c B u with c = (a - 1) / A (dt where A = 0) in place of dt B u. Then c replaces
// dt in dB and du (du = gp D + sum_n lam c B), the term's derivative in dt is dc/ddt = a, so
// ddt = sum_n lam a (h_{t-1} A + B u), and dA gains lam B u dc/dA (zoh_coef_dA_f); the adjoint
// recurrence is unchanged.
//
// Decomposition (as the forward kernel): a workgroup owns 64 channels of one batch, one channel
// per lane; wave w carries states w*S .. w*S+S-1 of the launch's block of at most 16 states
// (S <= 2). Larger N runs one launch per block of 16 states: per-state results (dB, dC, dA, dh0)
// belong to one block, and the per-(channel, step) sums over states (du, ddelta and, for the
// gate, sum_n C h) are added across the blocks in block order.
//   Phase 1: forward over 16-step segments, writing the state before each segment to the
//            workspace (the only stored states: N floats per channel per 16 steps).
//   Phase 2: segments in reverse. The workgroup computes the per-(channel, step) factors into
//            LDS; each wave reloads its segment's starting state, recomputes the segment's 16
//            states and decays in registers, then runs the reverse recurrence in two 8-step
//            halves. After each half, the per-(channel, step) sums over states go through LDS
//            (summed in wave order, like the forward's partial outputs) and the per-(state, step)
//            sums over the 64 channels of dB and dC are reduced in LDS and written as one partial
//            per workgroup.
//   A last kernel adds the partials in a fixed order: dB, dC over the channel groups, dA, dD,
//   dbias over the batch. Results are bitwise deterministic.
// B and C are first widened by a pre-pass into an fp32 copy in the workspace, rows padded with
// zeros to a multiple of 16 steps, so that a segment's values are aligned scalar loads.
#pragma once

#include "../../include/mamba_scan.h"
#include "bwd_layout.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace mscan {

struct BwdParams {
    const void* u;
    const void* delta;
    const void* z;
    const float* bc;  // fp32 B then C: (2, batch, N, lp)
    const float* A;
    const float* D;
    const float* bias;
    const float* h0;
    const float* dy;
    const float* dlast;
    float* du;
    float* ddelta;
    float* dz;
    float* dh0;
    float* ck;      // (batch, dim, nseg, ckn) this block's states before each segment
    float* bcpart;  // (groups, batch, 2, N, lp) dB / dC partials of each 64-channel group
    float* apart;   // (batch, dim, N)
    float* dpart;   // (batch, dim)
    float* bpart;   // (batch, dim)
    int64_t batch, dim, len, dstate, lp, nseg, groups;
    int64_t n0, nb, ckn;  // this launch's states n0 .. n0 + nb - 1; ck's state stride
    int64_t ck_n0;        // ck's state index of this block's first state
    int first, last;      // first / last block of states: initialises / finishes the sums
    int have_ck;          // ck holds the forward pass's states (all N): no recomputation
};

constexpr int kBwdW = 8;     // waves per workgroup
constexpr int kBwdSub = 8;   // steps per LDS exchange

typedef const __attribute__((address_space(4))) float* bwd_cptrf;

// Derivative of the zero-order-hold coefficient c = (e^{dt A} - 1) / A with respect to A, given
// x = dt * A, dA = e^x, c (from zoh_coef_f) and invA = 1 / A (0 where A = 0): (dt dA - c) / A,
// whose limit at A = 0 is dt^2 / 2. For |x| < 1/4 the Taylor series of the same function,
// dt^2 (1/2 + x/3 + x^2/8 + x^3/30 + x^4/144 + x^5/840) (the first dropped term, x^6 / 5760, is
// below 1e-7 of the sum there), so that two nearly equal terms are never subtracted; above it
// the closed form, whose cancellation costs at most a factor 2/|x| = 8 on the rounding of its
// terms. The derivative with respect to dt is dA itself.
__device__ __forceinline__ float zoh_coef_dA_f(float dt, float x, float dA, float c, float invA) {
    const float p = __builtin_fmaf(
        x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 840.0f, 1.0f / 144.0f), 1.0f / 30.0f), 0.125f),
                          1.0f / 3.0f),
        0.5f);
    const float small = dt * dt * p;
    const float big = __builtin_fmaf(dt, dA, -c) * invA;
    return __builtin_fabsf(x) < 0.25f ? small : big;
}

template <typename T>
__device__ __forceinline__ float load_el(const void* p, int64_t i) {
    return to_f32(static_cast<const T*>(p)[i]);
}

// MULTI: one of several blocks of states (first / last read from the parameters); otherwise the
// only block, with the sums over states finished in this launch.
// ZOH: B discretised by zero-order hold; the LDS factor F_DTU then holds u, the coefficient being
// per state.
template <typename T, int S, bool SOFTPLUS, bool HAS_Z, bool EXACT, bool MULTI, bool ZOH>
__global__ __launch_bounds__(64 * kBwdW) void scan_bwd_kernel(BwdParams p) {
    constexpr int W = kBwdW, SEG = kBwdSeg, SUB = kBwdSub;
    constexpr int QS = SEG / W;      // prologue steps per thread
    constexpr int ROWP = SEG + 4;    // LDS row of one channel's segment
    constexpr int SUBP = SUB + 1;    // LDS row of one channel's half-segment partials
    static_assert(S >= 1 && S <= 2 && QS == 2 && SUB == W, "backward tiling");
    enum { F_DT = 0, F_DTU, F_GP, F_U, F_SG, F_GZ, F_NUM };

    __shared__ float s_seg[F_NUM][64 * ROWP];   // per (channel, step) factors of the segment
    __shared__ float s_part[3][W * 64 * SUBP];  // per wave: sum lam B, sum q A, sum C h
    // [w][dB|dC][s][t] rows of the 64 lanes' values, padded so that consecutive rows start 4
    // banks apart: the channel sums below read one row per lane, 16 bytes at a time
    constexpr int REDP = 64 + 4;
    __shared__ __align__(16) float s_red[W * 2 * S * SUB * REDP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t b = blockIdx.x / p.groups;
    const int64_t grp = blockIdx.x - b * p.groups;
    const int64_t d0 = grp * 64;
    const int64_t L = p.len, N = p.dstate;
    const int nloc = wave * S;  // within the block
    const bool wave_live = EXACT || nloc < (int)p.nb;
    const int64_t nbase = p.n0 + (wave_live ? nloc : 0);
    const bool first = !MULTI || p.first, last = !MULTI || p.last;

    // prologue / epilogue role: row r = tid / 8; prologue steps 2k, 2k+1 of a segment,
    // epilogue step k of a half-segment (k = tid % 8)
    const int r = tid >> 3;
    const int k8 = tid & 7;
    const int64_t pd = d0 + r;
    const bool pvalid = pd < p.dim;
    const int64_t pdc = pvalid ? pd : 0;
    const int64_t prow = (b * p.dim + pdc) * L;
    const float pbias = p.bias ? p.bias[pdc] : 0.0f;
    const float pskip = p.D ? p.D[pdc] : 0.0f;

    // main role: this lane's channel, this wave's states
    const int64_t dm = d0 + lane;
    const bool mvalid = dm < p.dim;
    float a2[S], Av[S], ian[S], h[S], lam[S], gA[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        Av[s] = 0.0f;
        h[s] = 0.0f;
        lam[s] = 0.0f;
        gA[s] = 0.0f;
        if (wave_live && mvalid) {
            Av[s] = p.A[dm * N + nbase + s];
            if (p.h0) h[s] = p.h0[(b * p.dim + dm) * N + nbase + s];
            if (p.dlast) lam[s] = p.dlast[(b * p.dim + dm) * N + nbase + s];
        }
        a2[s] = Av[s] * kLog2e;
        ian[s] = Av[s] != 0.0f ? 1.0f / Av[s] : 0.0f;
    }
    // the input term of state s at step t: dt u B (Euler), or c u B with c the zero-order-hold
    // coefficient (cu = u then); the forward tiled kernel's arithmetic
    auto input_term = [&](int s, float dt, float cu, float a, float bb) __attribute__((always_inline)) {
        if constexpr (ZOH) return zoh_coef_f(dt, dt * Av[s], a, ian[s]) * cu * bb;
        return cu * bb;
    };
    const float* Brow = p.bc + (b * N + nbase) * p.lp;              // state nbase + s at + s*lp
    const float* Crow = p.bc + ((p.batch + b) * N + nbase) * p.lp;
    const int64_t ckn = p.ckn;
    float* ckrow = p.ck + (b * p.dim + (mvalid ? dm : 0)) * p.nseg * ckn + p.ck_n0 + (wave_live ? nloc : 0);

    // zero partials for waves that hold no states (read by the epilogue, never written after)
    if (!wave_live)
        for (int i = lane; i < 64 * SUBP; i += 64)
            for (int f = 0; f < 3; ++f) s_part[f][wave * 64 * SUBP + i] = 0.0f;

    // Raw inputs of a segment's prologue, fetched one segment ahead of their use. Step indices
    // are clamped into the row so every load is unconditional; steps past L are zeroed when used.
    auto tclamp = [&](int64_t t) __attribute__((always_inline)) { return t < 0 ? 0 : (t < L ? t : L - 1); };
    struct Raw1 {
        float x[QS], u[QS];
    };
    auto fetch1 = [&](int64_t k, Raw1& r) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            const int64_t t = tclamp(k * SEG + QS * k8 + j);
            r.x[j] = load_el<T>(p.delta, prow + t);
            r.u[j] = load_el<T>(p.u, prow + t);
        }
    };

    // ---- phase 1: forward, state before each segment to the workspace (skipped when the
    // forward pass saved them) ----
    Raw1 nx1;
    fetch1(0, nx1);
    for (int64_t k = 0; k < (p.have_ck ? 0 : p.nseg); ++k) {
        __syncthreads();
        const Raw1 r1 = nx1;
        fetch1(k + 1, nx1);
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            const int64_t t = k * SEG + QS * k8 + j;
            float dt = 0.0f, dtu = 0.0f;
            if (t < L) {
                const float x = r1.x[j] + pbias;
                dt = SOFTPLUS ? softplus_f(x) : hw_exp2(x * kLog2e);
                dtu = ZOH ? r1.u[j] : dt * r1.u[j];
            }
            s_seg[F_DT][r * ROWP + QS * k8 + j] = dt;
            s_seg[F_DTU][r * ROWP + QS * k8 + j] = dtu;
        }
        __syncthreads();
        if (wave_live) {
            if (mvalid)
#pragma unroll
                for (int s = 0; s < S; ++s) ckrow[k * ckn + s] = h[s];
            float bv[S][SEG];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const bwd_cptrf pb = (bwd_cptrf)(Brow + s * p.lp + k * SEG);
#pragma unroll
                for (int t = 0; t < SEG; ++t) bv[s][t] = pb[t];
            }
#pragma unroll
            for (int t = 0; t < SEG; ++t) {
                const float dt = s_seg[F_DT][lane * ROWP + t];
                const float dtu = s_seg[F_DTU][lane * ROWP + t];
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const float a = hw_exp2(dt * a2[s]);
                    h[s] = __builtin_fmaf(a, h[s], input_term(s, dt, dtu, a, bv[s][t]));
                }
            }
        }
    }

    // ---- phase 2: segments in reverse ----
    struct Raw2 {
        float x[QS], u[QS], gy[QS], z[QS];
    };
    auto fetch2 = [&](int64_t k, Raw2& r) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            const int64_t t = tclamp(k * SEG + QS * k8 + j);
            r.x[j] = load_el<T>(p.delta, prow + t);
            r.u[j] = load_el<T>(p.u, prow + t);
            r.gy[j] = p.dy[prow + t];
            r.z[j] = HAS_Z ? load_el<T>(p.z, prow + t) : 0.0f;
        }
    };
    float gDacc = 0.0f, gbacc = 0.0f;
    Raw2 nx2;
    fetch2(p.nseg - 1, nx2);
    for (int64_t k = p.nseg - 1; k >= 0; --k) {
        __syncthreads();
        const Raw2 r2 = nx2;
        fetch2(k - 1, nx2);
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            const int64_t t = k * SEG + QS * k8 + j;
            float dt = 0.0f, dtu = 0.0f, gp = 0.0f, uu = 0.0f, sg = 0.0f, gz = 0.0f;
            if (t < L && pvalid) {
                const float x = r2.x[j] + pbias;
                uu = r2.u[j];
                const float gy = r2.gy[j];
                if constexpr (SOFTPLUS) {
                    dt = softplus_f(x);
                    sg = hw_rcp(1.0f + hw_exp2(-x * kLog2e));
                } else {
                    dt = hw_exp2(x * kLog2e);
                }
                dtu = ZOH ? uu : dt * uu;
                if constexpr (HAS_Z) {
                    const float zz = r2.z[j];
                    const float sz = hw_rcp(1.0f + hw_exp2(-zz * kLog2e));
                    gp = gy * zz * sz;
                    gz = gy * (sz + zz * sz * (1.0f - sz));
                } else {
                    gp = gy;
                }
            } else if (t < L) {
                // rows past dim: same decay as row 0 would give, no gradient flowing in
                const float x = r2.x[j] + pbias;
                dt = SOFTPLUS ? softplus_f(x) : hw_exp2(x * kLog2e);
            }
            const int o = r * ROWP + QS * k8 + j;
            s_seg[F_DT][o] = dt;
            s_seg[F_DTU][o] = dtu;
            s_seg[F_GP][o] = gp;
            s_seg[F_U][o] = uu;
            s_seg[F_SG][o] = sg;
            s_seg[F_GZ][o] = gz;
        }
        __syncthreads();

        // recompute the segment's states and decays
        float hs[S], hseg[S][SEG], aseg[S][SEG], bv[S][SEG], cv[S][SEG], dtv[SEG], dtuv[SEG], gpv[SEG];
        if (wave_live) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                hs[s] = mvalid ? ckrow[k * ckn + s] : 0.0f;
                const bwd_cptrf pb = (bwd_cptrf)(Brow + s * p.lp + k * SEG);
                const bwd_cptrf pc = (bwd_cptrf)(Crow + s * p.lp + k * SEG);
#pragma unroll
                for (int t = 0; t < SEG; ++t) {
                    bv[s][t] = pb[t];
                    cv[s][t] = pc[t];
                }
            }
#pragma unroll
            for (int t = 0; t < SEG; ++t) {
                dtv[t] = s_seg[F_DT][lane * ROWP + t];
                dtuv[t] = s_seg[F_DTU][lane * ROWP + t];
                gpv[t] = s_seg[F_GP][lane * ROWP + t];
            }
#pragma unroll
            for (int s = 0; s < S; ++s) {
                float hh = hs[s];
#pragma unroll
                for (int t = 0; t < SEG; ++t) {
                    aseg[s][t] = hw_exp2(dtv[t] * a2[s]);
                    hh = __builtin_fmaf(aseg[s][t], hh, input_term(s, dtv[t], dtuv[t], aseg[s][t], bv[s][t]));
                    hseg[s][t] = hh;
                }
            }
        }

        // the segment's per-(channel, step) results and dB / dC sums, written once both halves are
        // done: a channel's 16 steps (64 bytes) by two adjacent stores instead of 32 bytes per half
        float o_u[2], o_x[2], o_z[2], o_bc[2];
        bool o_ok[2], o_bcok[2];
#pragma unroll
        for (int half = 1; half >= 0; --half) {
            o_ok[half] = false;
            o_bcok[half] = false;
            if (wave_live) {
                float gBc[S][SUB], gCc[S][SUB];
#pragma unroll
                for (int tt = SUB - 1; tt >= 0; --tt) {
                    const int t = half * SUB + tt;
                    float P1 = 0.0f, P2 = 0.0f, Y = 0.0f;
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        lam[s] = __builtin_fmaf(gpv[t], cv[s][t], lam[s]);
                        gCc[s][tt] = gpv[t] * hseg[s][t];
                        const float hp = t > 0 ? hseg[s][t - 1] : hs[s];
                        if constexpr (ZOH) {
                            // P1 = sum lam c B (du), P2 = sum lam a (h_{t-1} A + B u) (ddt)
                            const float x = dtv[t] * Av[s];
                            const float cf = zoh_coef_f(dtv[t], x, aseg[s][t], ian[s]);
                            const float lb = lam[s] * bv[s][t];
                            gBc[s][tt] = lam[s] * (cf * dtuv[t]);
                            P1 = __builtin_fmaf(lb, cf, P1);
                            const float la = lam[s] * aseg[s][t];
                            P2 = __builtin_fmaf(la, __builtin_fmaf(hp, Av[s], bv[s][t] * dtuv[t]), P2);
                            gA[s] = __builtin_fmaf(la * hp, dtv[t], gA[s]);
                            gA[s] = __builtin_fmaf(lb * dtuv[t], zoh_coef_dA_f(dtv[t], x, aseg[s][t], cf, ian[s]), gA[s]);
                        } else {
                            gBc[s][tt] = lam[s] * dtuv[t];
                            P1 = __builtin_fmaf(lam[s], bv[s][t], P1);
                            const float q = lam[s] * aseg[s][t] * hp;
                            P2 = __builtin_fmaf(q, Av[s], P2);
                            gA[s] = __builtin_fmaf(q, dtv[t], gA[s]);
                        }
                        Y = __builtin_fmaf(cv[s][t], hseg[s][t], Y);
                        lam[s] *= aseg[s][t];
                    }
                    const int o = (wave * 64 + lane) * SUBP + tt;
                    s_part[0][o] = P1;
                    s_part[1][o] = P2;
                    s_part[2][o] = Y;
                }
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int tt = 0; tt < SUB; ++tt) {
                        s_red[(((wave * 2 + 0) * S + s) * SUB + tt) * REDP + lane] = gBc[s][tt];
                        s_red[(((wave * 2 + 1) * S + s) * SUB + tt) * REDP + lane] = gCc[s][tt];
                    }
            }
            __syncthreads();
            // epilogue: step k8 of this half, channel r
            {
                const int tt = k8;
                const int64_t t = k * SEG + half * SUB + tt;
                float P1 = 0.0f, P2 = 0.0f, Y = 0.0f;
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const int o = (w * 64 + r) * SUBP + tt;
                    P1 += s_part[0][o];
                    P2 += s_part[1][o];
                    Y += s_part[2][o];
                }
                const int o = r * ROWP + half * SUB + tt;
                const float dt = s_seg[F_DT][o], gp = s_seg[F_GP][o], uu = s_seg[F_U][o];
                const float gdt = ZOH ? P2 : __builtin_fmaf(uu, P1, P2);
                const float gx = SOFTPLUS ? gdt * s_seg[F_SG][o] : gdt * dt;
                if (pvalid && t < L) {
                    // this block's share; earlier blocks' shares are already in the outputs
                    float gu = ZOH ? P1 : dt * P1, gxs = gx, ys = Y;
                    if (first) {
                        gu = __builtin_fmaf(gp, pskip, gu);
                        gDacc = __builtin_fmaf(gp, uu, gDacc);
                    } else {
                        gu += p.du[prow + t];
                        gxs += p.ddelta[prow + t];
                        if constexpr (HAS_Z) ys += p.dz[prow + t];
                    }
                    o_ok[half] = true;
                    o_u[half] = gu;
                    o_x[half] = gxs;
                    if constexpr (HAS_Z)  // sum_n C h until the last block, then the gate's gradient
                        o_z[half] = last ? s_seg[F_GZ][o] * __builtin_fmaf(pskip, uu, ys) : ys;
                    if (last) gbacc += gxs;  // dbias sums the finished ddelta
                }
            }
            // dB / dC of this half: one sum over the 64 channels per (dB|dC, state, step)
            if (tid < 2 * W * S * SUB) {
                const int tt = tid % SUB;
                const int s = (tid / SUB) % S;
                const int w = (tid / (SUB * S)) % W;
                const int q = tid / (SUB * S * W);
                const float* src = &s_red[(((w * 2 + q) * S + s) * SUB + tt) * REDP];
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < 64; i += 4) {
                    const float4 v = *reinterpret_cast<const float4*>(src + i);
                    acc += v.x;
                    acc += v.y;
                    acc += v.z;
                    acc += v.w;
                }
                o_bcok[half] = w * S + s < p.nb;
                o_bc[half] = acc;
            }
            __syncthreads();
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t t = k * SEG + half * SUB + k8;
            if (o_ok[half]) {
                p.du[prow + t] = o_u[half];
                p.ddelta[prow + t] = o_x[half];
                if constexpr (HAS_Z) p.dz[prow + t] = o_z[half];
            }
            if (o_bcok[half]) {
                const int tt = tid % SUB;
                const int s = (tid / SUB) % S;
                const int w = (tid / (SUB * S)) % W;
                const int q = tid / (SUB * S * W);
                p.bcpart[(((grp * p.batch + b) * 2 + q) * N + p.n0 + w * S + s) * p.lp + k * SEG + half * SUB + tt] =
                    o_bc[half];
            }
        }
    }

    // per-channel results: dh0, the batch's share of dA
    if (wave_live && mvalid) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int64_t i = (b * p.dim + dm) * N + nbase + s;
            if (p.dh0) p.dh0[i] = lam[s];
            p.apart[i] = gA[s];
        }
    }
    // the 8 threads of a channel add their dD and dbias shares
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
        gDacc += __shfl_xor(gDacc, off, 64);
        gbacc += __shfl_xor(gbacc, off, 64);
    }
    if (k8 == 0 && pvalid) {
        if (first) p.dpart[b * p.dim + pd] = gDacc;
        if (last) p.bpart[b * p.dim + pd] = gbacc;
    }
}

// B and C (any dtype, contiguous (batch, N, len)) widened into fp32 rows of length lp, zero past
// len. One thread per output element.
template <typename T>
__global__ __launch_bounds__(256) void bwd_bc_widen_kernel(const void* B, const void* C, float* out,
                                                           int64_t rows, int64_t len, int64_t lp) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= 2 * rows * lp) return;
    const int64_t row = i / lp, t = i - row * lp;
    const int64_t q = row / rows, rr = row - q * rows;
    out[i] = t < len ? load_el<T>(q ? C : B, rr * len + t) : 0.0f;
}

// ---------------------------------------------------------------------------------------------
// host side

inline int bwd_states_per_wave(int64_t nb) { return nb <= 8 ? 1 : 2; }

template <typename T, int S, bool SP, bool HZ, bool ZOH>
int launch_bwd_cfg(const BwdParams& q, hipStream_t stream) {
    void* args[] = {const_cast<BwdParams*>(&q)};
    const bool exact = q.nb == (int64_t)S * kBwdW;
    const bool multi = !(q.first && q.last);
    const void* fn =
        multi ? (exact ? reinterpret_cast<const void*>(&scan_bwd_kernel<T, S, SP, HZ, true, true, ZOH>)
                       : reinterpret_cast<const void*>(&scan_bwd_kernel<T, S, SP, HZ, false, true, ZOH>))
              : (exact ? reinterpret_cast<const void*>(&scan_bwd_kernel<T, S, SP, HZ, true, false, ZOH>)
                       : reinterpret_cast<const void*>(&scan_bwd_kernel<T, S, SP, HZ, false, false, ZOH>));
    return hipLaunchKernel(fn, dim3((unsigned)(q.batch * q.groups)), dim3(64 * kBwdW), args, 0, stream) ==
                   hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

template <typename T, int S, bool ZOH>
int launch_bwd_s(const BwdParams& q, bool softplus, hipStream_t stream) {
    const bool hz = q.z != nullptr;
    if (softplus && hz) return launch_bwd_cfg<T, S, true, true, ZOH>(q, stream);
    if (softplus) return launch_bwd_cfg<T, S, true, false, ZOH>(q, stream);
    if (hz) return launch_bwd_cfg<T, S, false, true, ZOH>(q, stream);
    return launch_bwd_cfg<T, S, false, false, ZOH>(q, stream);
}

template <typename T, bool ZOH>
int launch_bwd(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool softplus, hipStream_t stream) {
    const BwdLayout l = bwd_layout(s, p->checkpoints != nullptr);
    char* ws = static_cast<char*>(p->workspace);
    BwdParams q;
    q.u = p->u;
    q.delta = p->delta;
    q.z = p->z;
    q.bc = reinterpret_cast<const float*>(ws + l.off_bc);
    q.A = p->A;
    q.D = p->D;
    q.bias = p->delta_bias;
    q.h0 = p->h0;
    q.dy = p->dy;
    q.dlast = p->dlast_state;
    q.du = p->du;
    q.ddelta = p->ddelta;
    q.dz = p->dz;
    q.dh0 = p->dh0;
    q.ck = reinterpret_cast<float*>(ws + l.off_ck);
    q.bcpart = reinterpret_cast<float*>(ws + l.off_bcpart);
    q.apart = reinterpret_cast<float*>(ws + l.off_apart);
    q.dpart = reinterpret_cast<float*>(ws + l.off_dpart);
    q.bpart = reinterpret_cast<float*>(ws + l.off_bpart);
    q.batch = s.batch;
    q.dim = s.dim;
    q.len = s.len;
    q.dstate = s.dstate;
    q.lp = l.lp;
    q.nseg = l.nseg;
    q.groups = l.groups;

    const int64_t nwide = 2 * s.batch * s.dstate * l.lp;
    {
        const void* bsrc = p->B;
        const void* csrc = p->C;
        float* dst = reinterpret_cast<float*>(ws + l.off_bc);
        int64_t rows = s.batch * s.dstate, len = s.len, lp = l.lp;
        void* args[] = {&bsrc, &csrc, &dst, &rows, &len, &lp};
        if (hipLaunchKernel(reinterpret_cast<const void*>(&bwd_bc_widen_kernel<T>),
                            dim3((unsigned)((nwide + 255) / 256)), dim3(256), args, 0, stream) != hipSuccess)
            return MAMBA_SCAN_ERR_LAUNCH;
    }
    q.have_ck = p->checkpoints != nullptr;
    if (q.have_ck) q.ck = const_cast<float*>(p->checkpoints);
    q.ckn = q.have_ck ? s.dstate : bwd_block_states(s.dstate);
    for (int64_t n0 = 0; n0 < s.dstate; n0 += q.nb) {
        q.n0 = n0;
        q.ck_n0 = q.have_ck ? n0 : 0;
        int rc;
        if constexpr (ZOH) {
            // one state per wave, blocks of at most 8 states: with two, the coefficient and its
            // derivatives push the kernel past 256 VGPRs and about 100 of them spill to scratch
            // (3.8 ms per call at the Mamba-130m shape)
            q.nb = s.dstate - n0 > 8 ? 8 : s.dstate - n0;
            q.first = n0 == 0;
            q.last = n0 + q.nb == s.dstate;
            rc = launch_bwd_s<T, 1, true>(q, softplus, stream);
        } else {
            q.nb = bwd_next_block(s.dstate - n0);
            q.first = n0 == 0;
            q.last = n0 + q.nb == s.dstate;
            rc = bwd_states_per_wave(q.nb) == 1 ? launch_bwd_s<T, 1, false>(q, softplus, stream)
                                                : launch_bwd_s<T, 2, false>(q, softplus, stream);
        }
        if (rc != MAMBA_SCAN_OK) return rc;
    }
    BwdReduceParams r;
    r.bcpart = q.bcpart;
    r.apart = q.apart;
    r.dpart = q.dpart;
    r.bpart = q.bpart;
    r.dB = p->dB;
    r.dC = p->dC;
    r.dA = p->dA;
    r.dD = p->dD;
    r.dbias = p->ddelta_bias;
    r.batch = s.batch;
    r.dim = s.dim;
    r.len = s.len;
    r.dstate = s.dstate;
    r.lp = l.lp;
    r.groups = l.groups;
    return launch_bwd_reduce_any(r, stream);
}

}  // namespace mscan
