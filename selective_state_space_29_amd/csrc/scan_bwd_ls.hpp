// Lane-per-state backward pass for 16, 32 and 64 states (gfx950).
//
// The same gradients as the segment-tiled backward (scan_bwd.hpp: the derivative of the forward
// recurrence of "Mamba代码实战…" §3.1-§3.3 and §6, with the output contraction of "Mamba-minimal项目
// 解析…" 关键技术点 1 and the initial state of "手把手用PyTorch实现Mamba的SSM层…" §3.1), computed with the
// forward lane-per-state kernel's decomposition: one lane per (channel, state), a wave = 4
// channels x 16 states (lane 16c + n), a workgroup = W waves of one batch. The states are not
// kept from the forward pass, as "手把手用PyTorch实现Mamba的SSM层…" §4.2 prescribes: the state before
// every 16-step segment comes from the forward lane-per-state kernel (saved by the forward call,
// or written by a forward launch of the backward itself), and each segment's 16 states are
// recomputed from it with exactly the forward kernel's arithmetic, so bit for bit.
//
// Per segment, walked in reverse:
//   * Lane 16c + j computes the per-(channel, step) factors of step j of channel c (dt, dt u, the
//     gated output gradient gp = dy silu(z), sigmoid(x) for softplus', dy silu'(z)); the other
//     lanes of the row read them through the DPP row broadcast folded into the operation that
//     consumes them, as in the forward kernel.
//   * Forward: the segment's states and decays in registers, and C h into the wave's LDS area.
//   * Reverse, lam = dLoss/dh: lam += gp C; dC += gp h; dB += lam dt u; lam B and
//     q A with q = lam a h_{t-1} into LDS; dA += q dt; lam *= a.
//   * The three sums over states per (channel, step) (sum C h, sum lam B, sum q A) are read back
//     transposed, one step per lane, in state order; the lane then finishes du, ddelta, dz of its
//     step and accumulates its shares of dD and ddelta_bias.
//   * dB and dC are summed over the wave's 4 channels across its rows (v_permlane32_swap, then
//     v_permlane16_swap, each lane keeping a quarter of the sums), then over the workgroup's W
//     waves in LDS in wave order, and written as one partial per workgroup; a last kernel adds
//     the partials of the channel groups in a fixed order (and dA, dD, dbias over the batch):
//     deterministic.
// Per element 14 VALU operations (forward 4, reverse 10), about 2.8 for the sums over states and
// 3 for the channel sums; per (channel, step) about 35 for the factors and the finish.
// 32 and 64 states run one launch per block of 16 states, in order: each block's states are
// independent of the others' for dB, dC, dA and dh0; du, ddelta and (with a gate) the sum over
// states of C h are carried from block to block through the outputs, the last block finishing dz.
#pragma once

#include "../../include/mamba_scan.h"
#include "bwd_layout.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "scan_ls.hpp"

namespace mscan {

// Derivative in A of the zero-order-hold coefficient c = (e^{dt A} - 1) / A, from x = dt A,
// dA = e^x, c (zoh_coef2_f) and ia = 1 / A (0 where A = 0): (dt dA - c) / A, limit dt^2 / 2 at
// A = 0. Below |x| = 1/4 the Taylor series dt^2 (1/2 + x/3 + x^2/8 + x^3/30 + x^4/144 + x^5/840)
// (first dropped term under 1e-7 of the sum), above it the closed form (cancellation at most
// 2/|x| = 8).
__device__ __forceinline__ float zoh_coef_dA_x_f(float dt, float x, float dA, float c, float ia) {
    const float p = __builtin_fmaf(
        x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 840.0f, 1.0f / 144.0f), 1.0f / 30.0f), 0.125f),
                          1.0f / 3.0f),
        0.5f);
    const float small = dt * dt * p;
    const float big = __builtin_fmaf(dt, dA, -c) * ia;
    return __builtin_fabsf(x) < 0.25f ? small : big;
}

constexpr int kBlRowP = 20;                  // LDS floats per (channel, state) row of a segment
constexpr int kBlChanP = 16 * kBlRowP + 16;  // per channel: 16 rows, skewed by 16 banks
constexpr int kBlArea = 4 * kBlChanP;        // one quantity of a wave's 4 channels

struct BlsParams {
    const void* u;
    const void* delta;
    const void* z;
    const void* B;
    const void* C;
    const float* A;
    const float* D;
    const float* bias;
    const float* dy;
    const float* dlast;
    const float* ck;  // (batch, dim, nseg, 16): the state before every segment
    float* du;
    float* ddelta;
    float* dz;
    float* dh0;
    float* bcpart;  // (groups, batch, 2, N, lp) dB / dC partials of each channel group
    float* apart;   // (parts, batch, dim, N)
    float* dpart;   // (parts, batch, dim)
    float* bpart;   // (parts, batch, dim)
    float* carry;   // sub-parts 1 .. subs-1: (subs - 1, batch, dim, N) adjoint contributions,
                    // then as many decay products
    int64_t batch, dim, len, lp, nseg, groups;
    int64_t parts, spp;  // sequence parts; segments per part (the last part may have fewer)
    int64_t subs, sspp;  // the pre-pass's sub-parts (subs / parts to a part); segments per sub-part
    int64_t N, n0;    // dstate; this launch's states n0 .. n0 + 15
    int first, last;  // first / last block of 16 states: initialises / finishes the sums
};

template <int V>
struct BlIdx {
    static constexpr int value = V;
};

// f(BlIdx<I>{}) for I = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void bl_for(F&& f) {
    if constexpr (B < E) {
        f(BlIdx<B>{});
        bl_for<B + 1, E>(f);
    }
}

// Sequence parts: with p.parts > 1 workgroup (part, b, group) walks only the part's segments,
// part * spp .. (part + 1) * spp - 1. The reverse recurrence is linear in the adjoint it starts
// from, lam -> (lam + gp C) a per step, so a part's run over its steps from a zero adjoint gives
// a contribution R and its decays a product D such that the adjoint leaving the part is R + D lam
// for any entering lam. scan_bwd_ls_carry_kernel computes R and D for every sub-part of parts
// 1 .. P-1 (subs / P sub-parts tile a part), and part p starts from dlast folded through those of
// the sub-parts after it, last first. dh0 comes from part 0; the dA, dD and dbias partials are
// kept per part and added in part order by the reduction.
//
// MULTI: one of several blocks of 16 states (32 or 64 states): du, ddelta and, with a gate, the
// sum over states of C h are read back from the earlier blocks' launches and added to, in block
// order; the first block adds the skip term, the last one finishes dz. Otherwise the only block.
// ZOH: B discretised by zero-order hold. The input term is c u B with c = (e^{dt A} - 1) / A
// (zoh_coef2_f, the forward kernel's arithmetic; the row broadcast carries u): c replaces dt in dB
// and in the first sum over states (sum lam c B, du), the second becomes sum lam a (h A + B u)
// (ddt: dc/ddt = a), and dA gains lam B u dc/dA; c is recomputed in the reverse from the decay.
// With the zero-order hold the segment's coefficients are kept beside its states and decays and
// the kernel takes 221-250 VGPRs (the Euler one 164): 2 waves per SIMD instead of 3 (under the
// 168-VGPR cap of 3 about 100 of them spilled to scratch).
template <typename T, int W, bool SOFTPLUS, bool HAS_Z, bool MULTI, bool ZOH>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(ZOH ? 2 : 3)))
void scan_bwd_ls_kernel(BlsParams p) {
    __shared__ __align__(16) float s_w[W][2][kBlArea];    // per wave: two quantity areas
    __shared__ __align__(16) float s_bc[2][16 * kBlRowP];  // the segment's B | C: [state][step]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bg = p.batch * p.groups;
    const int64_t part = blockIdx.x / bg;
    const int64_t b = (blockIdx.x - part * bg) / p.groups;
    const int64_t grp = blockIdx.x - part * bg - b * p.groups;
    const int64_t d0 = grp * (4 * W) + wave * 4;
    const int c = lane >> 4, n = lane & 15;
    const bool valid = d0 + c < p.dim;
    const int64_t d = valid ? d0 + c : p.dim - 1;  // rows past dim: row dim-1's decay, no gradient
    const int64_t L = p.len;
    const int64_t nseg = p.nseg;
    const int64_t kbeg = part * p.spp, kend = kbeg + p.spp < nseg ? kbeg + p.spp : nseg;  // this part
    const int64_t NS = MULTI ? p.N : 16, n0 = MULTI ? p.n0 : 0;  // state count, this block's first
    const bool first = !MULTI || p.first, last = !MULTI || p.last;

    const float Av = p.A[d * NS + n0 + n];
    const float a2 = Av * kLog2e;
    const float ia = Av != 0.0f ? 1.0f / Av : 0.0f;  // zero-order hold only
    const float bias = p.bias ? p.bias[d] : 0.0f;
    const float Dv = p.D ? p.D[d] : 0.0f;
    const int64_t si = (b * p.dim + d) * NS + n0 + n;  // this lane's (b, d, state)
    float lam = (p.dlast && valid) ? p.dlast[si] : 0.0f;
    if (valid) {
        // the adjoint entering this part: dlast carried through the later sub-parts, last first
        // (rows past dim keep a zero adjoint: their dB / dC terms must vanish)
        const int64_t pstride = p.batch * p.dim * NS;
        const float* const dprod = p.carry + (p.subs - 1) * pstride;
        const int64_t gend = (part + 1) * (p.subs / p.parts);  // the first sub-part after this part
        for (int64_t g = p.subs - 1; g >= gend; --g)
            lam = __builtin_fmaf(dprod[(g - 1) * pstride + si], lam, p.carry[(g - 1) * pstride + si]);
    }
    float gA = 0.0f, accD = 0.0f, accX = 0.0f;

    // Buffer descriptors with 32-bit byte offsets (the host checks that they fit): the wave's 4
    // rows of u / delta / z / dy / du / ddelta / dz and of the saved states, the batch's B / C;
    // the segment's offset is an SGPR. Past len, loads read finite values of the next row (or 0
    // past the range) that the step mask below discards; stores there get an offset past the
    // range and are dropped.
    constexpr uint32_t es = sizeof(T);
    const int64_t d0c = d0 < p.dim ? d0 : p.dim - 1;
    const int64_t dl = d0 + 3 < p.dim ? d0 + 3 : p.dim - 1;
    const uint32_t dr = (uint32_t)(d - d0c);
    const int64_t row0 = b * p.dim + d0c, nrows = dl - d0c + 1;
    auto rows_rsrc = [&](const void* base, int64_t e) __attribute__((always_inline)) {
        char* p0 = const_cast<char*>(static_cast<const char*>(base)) + row0 * L * e;
        return __builtin_amdgcn_make_buffer_rsrc(p0, 0, (int)(nrows * L * e), kLsWord3);
    };
    const __amdgpu_buffer_rsrc_t ur = rows_rsrc(p.u, es), xr = rows_rsrc(p.delta, es);
    const __amdgpu_buffer_rsrc_t zr = HAS_Z ? rows_rsrc(p.z, es) : ur;
    const __amdgpu_buffer_rsrc_t gr = rows_rsrc(p.dy, 4);
    const __amdgpu_buffer_rsrc_t our = rows_rsrc(p.du, 4), oxr = rows_rsrc(p.ddelta, 4);
    const __amdgpu_buffer_rsrc_t ozr = HAS_Z ? rows_rsrc(p.dz, 4) : our;
    const __amdgpu_buffer_rsrc_t ckr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.ck) + row0 * nseg * NS, 0, (int)(nrows * nseg * NS * 4), kLsWord3);
    const uint32_t oi = (dr * (uint32_t)L + n) * es;  // this lane's step n of a segment, inputs
    const uint32_t of = (dr * (uint32_t)L + n) * 4u;  // and fp32 rows
    const uint32_t ock = (dr * (uint32_t)(nseg * NS) + (uint32_t)(n0 + n)) * 4u;

    auto load_el = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff) __attribute__((always_inline)) {
        if constexpr (sizeof(T) == 2)
            return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, (int)soff, 0);
        else
            return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, (int)soff, 0);
    };
    auto widen = [](uint32_t v) __attribute__((always_inline)) {
        return __uint_as_float(sizeof(T) == 2 ? v << 16 : v);
    };

    // B / C staging: threads 0..255, two steps of one (B|C, state) row each; B|C wave-uniform
    const bool stager = tid < 256;
    const int sq = (wave >> 1) & 1, sn = (tid >> 3) & 15, st = (tid & 7) * 2;  // sq wave-uniform
    const __amdgpu_buffer_rsrc_t bcr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(sq ? p.C : p.B)) + (b * NS + n0) * L * es, 0, (int)(16 * L * es),
        kLsWord3);
    const uint32_t obc = (uint32_t)(sn * L + st) * es;
    float* const sdst = &s_bc[sq][sn * kBlRowP + st];
    auto stage_fetch = [&](int64_t k, uint32_t (&v)[2]) __attribute__((always_inline)) {
        const uint32_t so = (uint32_t)(k * 16) * es;
        v[0] = load_el(bcr, obc, so);
        v[1] = load_el(bcr, obc + es, so);
    };
    auto stage_store = [&](const uint32_t (&v)[2]) __attribute__((always_inline)) {
        *reinterpret_cast<float2*>(sdst) = float2{widen(v[0]), widen(v[1])};
    };

    // raw inputs of this lane's step of a segment, and its state's saved value, one segment ahead
    // (MULTI: also the earlier blocks' du, ddelta and sum of C h of this step, read whether or
    // not this is the first block, which does not use them: no branch around the loads)
    struct Raw {
        uint32_t x, u, z, g, h, pu, px, pz;
    };
    auto fetch = [&](int64_t k, Raw& w) __attribute__((always_inline)) {
        const uint32_t so = (uint32_t)(k * 16) * es, s4 = (uint32_t)(k * 64);
        w.x = load_el(xr, oi, so);
        w.u = load_el(ur, oi, so);
        w.z = HAS_Z ? load_el(zr, oi, so) : 0u;
        w.g = __builtin_amdgcn_raw_buffer_load_b32(gr, (int)of, (int)s4, 0);
        w.h = __builtin_amdgcn_raw_buffer_load_b32(ckr, (int)ock, (int)(k * NS * 4), 0);
        if constexpr (MULTI) {
            w.pu = __builtin_amdgcn_raw_buffer_load_b32(our, (int)of, (int)s4, 0);
            w.px = __builtin_amdgcn_raw_buffer_load_b32(oxr, (int)of, (int)s4, 0);
            w.pz = HAS_Z ? __builtin_amdgcn_raw_buffer_load_b32(ozr, (int)of, (int)s4, 0) : 0u;
        } else {
            w.pu = w.px = w.pz = 0u;
        }
    };

    float* const area0 = &s_w[wave][0][0];
    float* const area1 = &s_w[wave][1][0];
    float* const row0p = area0 + c * kBlChanP + n * kBlRowP;  // this lane's (channel, state) rows
    float* const row1p = area1 + c * kBlChanP + n * kBlRowP;
    const float* const col0 = area0 + c * kBlChanP + n;  // step n of channel c, state m at m * kBlRowP
    const float* const col1 = area1 + c * kBlChanP + n;
    auto col_sum = [](const float* col) __attribute__((always_inline)) {
        float s = col[0];
#pragma unroll
        for (int m = 1; m < 16; ++m) s += col[m * kBlRowP];
        return s;
    };

    // per-(channel, step) factors of this lane's step of segment k (the forward kernel's dt and
    // dt u, bit for bit)
    struct Fac {
        float dt, dtu, gp, uu, sg, gz, h, pu, px, pz;
    };
    auto factors = [&](const Raw& w, int64_t k) __attribute__((always_inline)) {
        Fac f;
        const bool live = k * 16 + n < L;
        const float xb = widen(w.x) + bias;
        const float x = live ? xb : -__builtin_inff();  // past len: dt = 0, the state carried
        f.uu = widen(w.u);
        const float gy = (live && valid) ? __uint_as_float(w.g) : 0.0f;
        if constexpr (SOFTPLUS) {
            f.dt = softplus_f(x);
            f.sg = hw_rcp(1.0f + hw_exp2(-x * kLog2e));
        } else {
            f.dt = hw_exp2(x * kLog2e);
            f.sg = 0.0f;
        }
        f.dtu = ZOH ? f.uu : f.dt * f.uu;
        if constexpr (HAS_Z) {
            const float zz = widen(w.z);
            const float sz = hw_rcp(1.0f + hw_exp2(-zz * kLog2e));
            f.gp = gy * zz * sz;
            f.gz = gy * (sz + zz * sz * (1.0f - sz));
        } else {
            f.gp = gy;
            f.gz = 0.0f;
        }
        f.h = __uint_as_float(w.h);
        f.pu = __uint_as_float(w.pu);
        f.px = __uint_as_float(w.px);
        f.pz = __uint_as_float(w.pz);
        return f;
    };

    // Software pipeline: segment k-1's raw inputs and B / C are loaded at the top of segment k
    // and turned into values before segment k's stores, so no wait for them covers a store.
    Raw raw;
    fetch(kend - 1, raw);
    uint32_t sv[2];
    if (stager) {
        stage_fetch(kend - 1, sv);
        stage_store(sv);
    }
    Fac cur = factors(raw, kend - 1);
    for (int64_t k = kend - 1; k >= kbeg; --k) {
        __syncthreads();  // the segment's B / C staged; the previous segment's LDS reads done
        const uint32_t s4 = (uint32_t)(k * 64);
        const bool live = k * 16 + n < L;
        const int64_t kp = k > kbeg ? k - 1 : kbeg;
        fetch(kp, raw);
        if (stager) stage_fetch(kp, sv);
        const float dt = cur.dt, dtu = cur.dtu, gp = cur.gp;
        float Bv[16], Cv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 vb = *reinterpret_cast<const float4*>(&s_bc[0][n * kBlRowP + 4 * q]);
            const float4 vc = *reinterpret_cast<const float4*>(&s_bc[1][n * kBlRowP + 4 * q]);
            Bv[4 * q] = vb.x, Bv[4 * q + 1] = vb.y, Bv[4 * q + 2] = vb.z, Bv[4 * q + 3] = vb.w;
            Cv[4 * q] = vc.x, Cv[4 * q + 1] = vc.y, Cv[4 * q + 2] = vc.z, Cv[4 * q + 3] = vc.w;
        }

        // forward over the segment from its saved state: hp[j] = state before step j
        float hp[16], dA[16], cfs[ZOH ? 16 : 1];
        float h = cur.h;
        {
            float yv[4];
            bl_for<0, 16>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                hp[j] = h;
                if constexpr (ZOH) {
                    const float dtb = row_bcast<j>(dt);
                    const float x2 = dtb * a2;
                    dA[j] = hw_exp2(x2);
                    cfs[j] = zoh_coef2_f(dtb, x2, dA[j], ia);
                    h = __builtin_fmaf(dA[j], h, cfs[j] * row_bcast<j>(dtu) * Bv[j]);
                } else {
                    dA[j] = hw_exp2(row_bcast<j>(dt) * a2);
                    h = __builtin_fmaf(dA[j], h, row_bcast<j>(dtu) * Bv[j]);
                }
                yv[j % 4] = Cv[j] * h;
                if constexpr (j % 4 == 3)
                    *reinterpret_cast<float4*>(row0p + (j - 3)) = float4{yv[0], yv[1], yv[2], yv[3]};
            });
        }
        const float hend = h;
        __builtin_amdgcn_wave_barrier();
        const float Ys = col_sum(col0);  // sum_n C h of step n
        __builtin_amdgcn_wave_barrier();

        // reverse over the segment
        float dBp[16], dCp[16];
        {
            float p1[4], p2[4];
            bl_for<0, 16>([&](auto ic) __attribute__((always_inline)) {
                constexpr int j = 15 - decltype(ic)::value;
                const float hs = j == 15 ? hend : hp[j < 15 ? j + 1 : 15];  // state after step j
                const float gpb = row_bcast<j>(gp);
                lam = __builtin_fmaf(gpb, Cv[j], lam);
                dCp[j] = gpb * hs;
                if constexpr (ZOH) {
                    const float dtb = row_bcast<j>(dt), ub = row_bcast<j>(dtu);
                    const float cf = cfs[j];
                    dBp[j] = lam * (cf * ub);
                    const float lb = lam * Bv[j];
                    p1[j % 4] = lb * cf;
                    const float la = lam * dA[j];
                    p2[j % 4] = la * __builtin_fmaf(hp[j], Av, Bv[j] * ub);
                    gA = __builtin_fmaf(la * hp[j], dtb, gA);
                    gA = __builtin_fmaf(lb * ub, zoh_coef_dA_x_f(dtb, dtb * Av, dA[j], cf, ia), gA);
                } else {
                    dBp[j] = lam * row_bcast<j>(dtu);
                    p1[j % 4] = lam * Bv[j];
                    const float q = lam * dA[j] * hp[j];
                    p2[j % 4] = q * Av;
                    gA = __builtin_fmaf(q, row_bcast<j>(dt), gA);
                }
                lam *= dA[j];
                if constexpr (j % 4 == 0) {
                    *reinterpret_cast<float4*>(row0p + j) = float4{p1[0], p1[1], p1[2], p1[3]};
                    *reinterpret_cast<float4*>(row1p + j) = float4{p2[0], p2[1], p2[2], p2[3]};
                }
            });
        }
        __builtin_amdgcn_wave_barrier();
        const float P1 = col_sum(col0);  // sum_n lam B (zero-order hold: sum_n lam c B)
        const float P2 = col_sum(col1);  // sum_n lam a h_{t-1} A (zero-order hold: + lam a B u)
        __builtin_amdgcn_wave_barrier();

        // dB / dC over the wave's 4 channels (rows), reduce-scattered across the rows: rows r and
        // r + 2 added by v_permlane32_swap (lower half keeps dB, upper half dC), then rows r and
        // r ^ 1 by v_permlane16_swap (even rows keep steps 0-7, odd rows steps 8-15). Lane 16r + n
        // ends with the 4-channel sums of state n, quantity r / 2, steps 8 (r % 2) .. + 7.
        float s1[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dBp[j]), __float_as_uint(dCp[j]), false, false);
            s1[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        float s2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(s1[j]), __float_as_uint(s1[j + 8]), false, false);
            s2[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        // the wave's sums, [dB|dC][state][step], for the workgroup's sum below (after the column
        // reads of area1 above: a wave's LDS accesses are performed in order)
        __builtin_amdgcn_wave_barrier();
        {
            float* const ws = area1 + (c >> 1) * 256 + n * 16 + (c & 1) * 8;
            *reinterpret_cast<float4*>(ws) = float4{s2[0], s2[1], s2[2], s2[3]};
            *reinterpret_cast<float4*>(ws + 4) = float4{s2[4], s2[5], s2[6], s2[7]};
        }

        // the next segment's values (its loads issued at the top), before this segment's stores
        const Fac nxt = factors(raw, kp);
        const float2 bcn = float2{widen(sv[0]), widen(sv[1])};

        // finish step n of channel c
        {
            const float uu = cur.uu;
            const float gdt = ZOH ? P2 : __builtin_fmaf(uu, P1, P2);
            const float gin = ZOH ? P1 : dt * P1;  // the input term's share of du
            float gx = SOFTPLUS ? gdt * cur.sg : gdt * dt;
            float gu = first ? __builtin_fmaf(gp, Dv, gin) : gin + cur.pu;
            float ys = Ys;
            if constexpr (MULTI) {
                if (!first) {
                    gx += cur.px;
                    ys += cur.pz;
                }
            }
            if (live) {
                if (first) accD = __builtin_fmaf(gp, uu, accD);
                if (last) accX += gx;  // dbias sums the finished ddelta
            }
            const bool st_ok = live && valid;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gu), our, (int)(st_ok ? of : kLsDropBase), (int)s4, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gx), oxr, (int)(st_ok ? of : kLsDropBase), (int)s4, 0);
            if constexpr (HAS_Z) {
                // the sum over states of C h until the last block, then the gate's gradient
                const float gzo = last ? cur.gz * __builtin_fmaf(Dv, uu, ys) : ys;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gzo), ozr, (int)(st_ok ? of : kLsDropBase), (int)s4, 0);
            }
        }
        __syncthreads();  // every wave's dB / dC sums written; every wave done with s_bc
        if (stager) {
            // dB / dC of the workgroup: the W waves' sums in wave order, one partial per group
            const int e = sq * 256 + sn * 16 + st;
            float2 acc = *reinterpret_cast<const float2*>(&s_w[0][1][e]);
#pragma unroll
            for (int w = 1; w < W; ++w) {
                const float2 v = *reinterpret_cast<const float2*>(&s_w[w][1][e]);
                acc.x += v.x;
                acc.y += v.y;
            }
            *reinterpret_cast<float2*>(p.bcpart + (((grp * p.batch + b) * 2 + sq) * NS + n0 + sn) * p.lp + k * 16 + st) = acc;
            *reinterpret_cast<float2*>(sdst) = bcn;  // the next segment's B / C
        }
        cur = nxt;
    }

    if (valid) {
        if (p.dh0 && part == 0) p.dh0[si] = lam;
        p.apart[part * p.batch * p.dim * NS + si] = gA;
    }
    // the channel's dD and dbias shares: its 16 lanes (one step of every segment each)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        accD += __shfl_xor(accD, off, 64);
        accX += __shfl_xor(accX, off, 64);
    }
    if (n == 0 && valid) {
        if (first) p.dpart[(part * p.batch + b) * p.dim + d] = accD;
        if (last) p.bpart[(part * p.batch + b) * p.dim + d] = accX;
    }
}

// Sub-parts of parts 1 .. parts-1 of the sequence (above): each lane (channel, state) runs the
// reverse adjoint recurrence over its sub-part's steps from zero, lam -> a lam + a gp C (dt, gp and a computed
// as in the main kernel; one FMA per step on the dependent chain), and writes the contribution lam
// and the sub-part's decay product exp(A * sum of its dt), capped at FLT_MAX (an overflowing product
// times a zero adjoint must stay zero, as in the sequential recurrence). A workgroup is one wave
// (4 channels of one batch) that stages the segment's C in its own LDS, one segment ahead: no
// workgroup barrier (a wave's LDS accesses are performed in order).
template <typename T, bool SOFTPLUS, bool HAS_Z>
__global__ __launch_bounds__(64) void scan_bwd_ls_carry_kernel(BlsParams p) {
    __shared__ __align__(16) float s_c[2][16 * kBlRowP];  // [buffer][state][step]

    const int lane = threadIdx.x & 63;
    const int64_t cg = (p.dim + 3) / 4;  // 4-channel groups
    const int64_t bg = p.batch * cg;
    const int64_t g0 = p.subs / p.parts;  // sub-parts to a part; part 0's need none
    const int64_t sub = g0 + blockIdx.x / bg;
    const int64_t b = (blockIdx.x - (sub - g0) * bg) / cg;
    const int64_t d0 = (blockIdx.x - (sub - g0) * bg - b * cg) * 4;
    const int c = lane >> 4, n = lane & 15;
    const bool valid = d0 + c < p.dim;
    const int64_t d = valid ? d0 + c : p.dim - 1;
    const int64_t L = p.len;
    const int64_t NS = p.N, n0 = p.n0;
    // segments kbeg .. kend-1 within the part (an empty sub-part: contribution 0, product 1)
    const int64_t pbeg = (sub / g0) * p.spp;
    const int64_t pend = pbeg + p.spp < p.nseg ? pbeg + p.spp : p.nseg;
    const int64_t kbeg = pbeg + (sub % g0) * p.sspp;
    const int64_t kend = kbeg + p.sspp < pend ? kbeg + p.sspp : pend;

    const float a2 = p.A[d * NS + n0 + n] * kLog2e;
    const float bias = p.bias ? p.bias[d] : 0.0f;

    constexpr uint32_t es = sizeof(T);
    const int64_t dl = d0 + 3 < p.dim ? d0 + 3 : p.dim - 1;
    const uint32_t dr = (uint32_t)(d - d0);
    const int64_t row0 = b * p.dim + d0, nrows = dl - d0 + 1;
    auto rows_rsrc = [&](const void* base, int64_t e) __attribute__((always_inline)) {
        char* p0 = const_cast<char*>(static_cast<const char*>(base)) + row0 * L * e;
        return __builtin_amdgcn_make_buffer_rsrc(p0, 0, (int)(nrows * L * e), kLsWord3);
    };
    const __amdgpu_buffer_rsrc_t xr = rows_rsrc(p.delta, es);
    const __amdgpu_buffer_rsrc_t zr = HAS_Z ? rows_rsrc(p.z, es) : xr;
    const __amdgpu_buffer_rsrc_t gr = rows_rsrc(p.dy, 4);
    const uint32_t oi = (dr * (uint32_t)L + n) * es, of = (dr * (uint32_t)L + n) * 4u;
    // C staging: lane l stages steps 4 (l % 4) .. + 3 of state row l / 4 (past len: the next
    // row's values or 0, at steps whose dt and gp are zero)
    const int sn = lane >> 2, st = (lane & 3) * 4;
    const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(p.C)) + (b * NS + n0) * L * es, 0, (int)(16 * L * es), kLsWord3);
    const uint32_t oc = (uint32_t)(sn * L + st) * es;
    auto load_el = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff) __attribute__((always_inline)) {
        if constexpr (sizeof(T) == 2)
            return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, (int)soff, 0);
        else
            return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, (int)soff, 0);
    };
    auto widen = [](uint32_t v) __attribute__((always_inline)) {
        return __uint_as_float(sizeof(T) == 2 ? v << 16 : v);
    };

    struct Raw {
        uint32_t x, z, g, c[4];
    };
    auto fetch = [&](int64_t k, Raw& w) __attribute__((always_inline)) {
        const uint32_t so = (uint32_t)(k * 16) * es, s4 = (uint32_t)(k * 64);
        w.x = load_el(xr, oi, so);
        w.z = HAS_Z ? load_el(zr, oi, so) : 0u;
        w.g = __builtin_amdgcn_raw_buffer_load_b32(gr, (int)of, (int)s4, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) w.c[j] = load_el(cr, oc + j * es, so);
    };
    auto stage = [&](const Raw& w, int buf) __attribute__((always_inline)) {
        *reinterpret_cast<float4*>(&s_c[buf][sn * kBlRowP + st]) =
            float4{widen(w.c[0]), widen(w.c[1]), widen(w.c[2]), widen(w.c[3])};
    };
    // dt and gp of this lane's step of segment k, as the main kernel computes them
    auto factors = [&](const Raw& w, int64_t k, float& dt, float& gp) __attribute__((always_inline)) {
        const bool live = k * 16 + n < L;
        const float xb = widen(w.x) + bias;
        const float x = live ? xb : -__builtin_inff();
        dt = SOFTPLUS ? softplus_f(x) : hw_exp2(x * kLog2e);
        const float gy = (live && valid) ? __uint_as_float(w.g) : 0.0f;
        if constexpr (HAS_Z) {
            const float zz = widen(w.z);
            gp = gy * zz * hw_rcp(1.0f + hw_exp2(-zz * kLog2e));
        } else {
            gp = gy;
        }
    };

    Raw raw;
    fetch(kend - 1, raw);
    stage(raw, 0);
    float dt, gp;
    factors(raw, kend - 1, dt, gp);
    float lam = 0.0f, sdt = 0.0f;  // sdt: this lane's steps' dt summed (its row sums the channel's)
    int buf = 0;
    for (int64_t k = kend - 1; k >= kbeg; --k) {
        const int64_t kp = k > kbeg ? k - 1 : kbeg;
        fetch(kp, raw);
        __builtin_amdgcn_wave_barrier();
        float Cv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 vc = *reinterpret_cast<const float4*>(&s_c[buf][n * kBlRowP + 4 * q]);
            Cv[4 * q] = vc.x, Cv[4 * q + 1] = vc.y, Cv[4 * q + 2] = vc.z, Cv[4 * q + 3] = vc.w;
        }
        sdt += dt;
        bl_for<0, 16>([&](auto ic) __attribute__((always_inline)) {
            constexpr int j = 15 - decltype(ic)::value;
            const float a = hw_exp2(row_bcast<j>(dt) * a2);
            lam = __builtin_fmaf(a, lam, a * (row_bcast<j>(gp) * Cv[j]));
        });
        // the next segment's C into the other buffer (this wave's reads of it are done: in order)
        __builtin_amdgcn_wave_barrier();
        stage(raw, buf ^ 1);
        factors(raw, kp, dt, gp);
        buf ^= 1;
    }
    // the channel's sum of dt over the part: the row's 16 lanes
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) sdt += __shfl_xor(sdt, off, 64);
    if (valid) {
        const int64_t pstride = p.batch * p.dim * NS;
        const int64_t i = (sub - 1) * pstride + (b * p.dim + d) * NS + n0 + n;
        p.carry[i] = lam;
        p.carry[(p.subs - 1) * pstride + i] = __builtin_fminf(hw_exp2(a2 * sdt), 3.4028234663852886e38f);
    }
}

// ---------------------------------------------------------------------------------------------
// host side

template <typename T, bool SP, bool HZ, bool ZOH>
int launch_bwd_ls_cfg(const BlsParams& q, hipStream_t stream) {
    void* args[] = {const_cast<BlsParams*>(&q)};
    if (q.parts > 1) {
        // the adjoint contribution and decay product of every sub-part after part 0, before the
        // parts run
        const void* cf = reinterpret_cast<const void*>(&scan_bwd_ls_carry_kernel<T, SP, HZ>);
        const int64_t nsub = q.subs - q.subs / q.parts;
        if (hipLaunchKernel(cf, dim3((unsigned)(nsub * q.batch * ((q.dim + 3) / 4))), dim3(64), args, 0, stream) !=
            hipSuccess)
            return MAMBA_SCAN_ERR_LAUNCH;
    }
    const void* fn = q.N > 16 ? reinterpret_cast<const void*>(&scan_bwd_ls_kernel<T, kBlsW, SP, HZ, true, ZOH>)
                              : reinterpret_cast<const void*>(&scan_bwd_ls_kernel<T, kBlsW, SP, HZ, false, ZOH>);
    return hipLaunchKernel(fn, dim3((unsigned)(q.parts * q.batch * q.groups)), dim3(64 * kBlsW), args, 0, stream) ==
                   hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

template <typename T, bool ZOH>
int launch_bwd_ls(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool softplus, hipStream_t stream) {
    if (!bwd_ls_fits(s, sizeof(T))) return MAMBA_SCAN_ERR_UNSUPPORTED;
    const bool given = p->checkpoints != nullptr;
    const BwdLayout l = bwd_ls_layout(s, given);
    char* ws = static_cast<char*>(p->workspace);
    float* ck = given ? const_cast<float*>(p->checkpoints) : reinterpret_cast<float*>(ws + l.off_ck);
    const int64_t L = s.len, DL = s.dim * L, N = s.dstate;
    if (!given) {
        // the state before every segment, written by the forward kernel that a forward call saving
        // them runs (lane-per-state or chunked: the same bits); its y goes to du, which the
        // backward overwrites
        ScanParams f{};
        f.u = p->u;
        f.delta = p->delta;
        f.z = p->z;
        f.B = p->B;
        f.C = p->C;
        f.A = p->A;
        f.D = p->D;
        f.bias = p->delta_bias;
        f.h0 = p->h0;
        f.y = p->du;
        f.last_state = nullptr;
        f.batch = s.batch;
        f.dim = s.dim;
        f.len = L;
        f.dstate = N;
        f.su_b = f.sdt_b = f.sz_b = f.sy_b = DL;
        f.su_d = f.sdt_d = f.sz_d = f.sy_d = L;
        f.sB_b = f.sC_b = N * L;
        f.sB_n = f.sC_n = L;
        f.sh0_b = s.dim * N;
        f.sh0_d = N;
        f.sA_d = N;
        f.sD = f.sbias = 1;
        f.softplus = softplus ? 1 : 0;
        f.zoh_b = ZOH ? 1 : 0;
        f.ck = ck;
        f.ck_nseg = l.nseg;
        const int rc = launch_fwd_checkpoints(f, sizeof(T) == 2, stream);
        if (rc != MAMBA_SCAN_OK) return rc;
    }
    BlsParams q;
    q.u = p->u;
    q.delta = p->delta;
    q.z = p->z;
    q.B = p->B;
    q.C = p->C;
    q.A = p->A;
    q.D = p->D;
    q.bias = p->delta_bias;
    q.dy = p->dy;
    q.dlast = p->dlast_state;
    q.ck = ck;
    q.du = p->du;
    q.ddelta = p->ddelta;
    q.dz = p->dz;
    q.dh0 = p->dh0;
    q.bcpart = reinterpret_cast<float*>(ws + l.off_bcpart);
    q.apart = reinterpret_cast<float*>(ws + l.off_apart);
    q.dpart = reinterpret_cast<float*>(ws + l.off_dpart);
    q.bpart = reinterpret_cast<float*>(ws + l.off_bpart);
    q.carry = reinterpret_cast<float*>(ws + l.off_carry);
    q.parts = l.parts;
    q.spp = l.spp;
    q.subs = l.subs;
    q.sspp = l.sspp;
    q.batch = s.batch;
    q.dim = s.dim;
    q.len = L;
    q.lp = l.lp;
    q.nseg = l.nseg;
    q.groups = l.groups;
    q.N = N;
    const bool hz = p->z != nullptr;
    // one launch per block of 16 states, in order (the sums over states carried in du, ddelta, dz)
    for (int64_t n0 = 0; n0 < N; n0 += 16) {
        q.n0 = n0;
        q.first = n0 == 0;
        q.last = n0 + 16 == N;
        const int rc = softplus ? (hz ? launch_bwd_ls_cfg<T, true, true, ZOH>(q, stream)
                                      : launch_bwd_ls_cfg<T, true, false, ZOH>(q, stream))
                                : (hz ? launch_bwd_ls_cfg<T, false, true, ZOH>(q, stream)
                                      : launch_bwd_ls_cfg<T, false, false, ZOH>(q, stream));
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
    r.len = L;
    r.dstate = N;
    r.lp = l.lp;
    r.groups = l.groups;
    r.parts = l.parts;
    return launch_bwd_reduce_any(r, stream);
}

}  // namespace mscan
