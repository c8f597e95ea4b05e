// Chunked (L-parallel) lane-per-state forward kernel for 16 states (gfx950).
//
// The same operation as the other kernels (the recurrence of "Mamba代码实战…" §3.1-§3.3 and §6,
// the output contraction of "Mamba-minimal项目解析…" 关键技术点 1, the optional initial state of
// "手把手用PyTorch实现Mamba的SSM层…" §3.1), parallel along the sequence as well: a wave holds ONE
// channel, lane 16 r + n = state n of run r, and the 4 rows of the wave scan 4 consecutive runs
// of K steps of each 4K-step chunk at the same time.
//   * Local pass: each lane runs its state's recurrence over its run from a zero state, keeping
//     every step's decay dA and input term dt u B in registers; its run's pair (a, b) is then
//     a = product of the run's decays = exp(A * sum of the run's dt) and b = the run's end state.
//   * Combine: the pairs of the 4 runs are combined across the rows with the associative
//     operator of the parallel scan of "手把手用PyTorch实现Mamba的SSM层…" §3.2,
//     (a1, b1) then (a2, b2) = (a1 a2, a2 b1 + b2), by two cross-row exchanges
//     (v_permlane16_swap: row pairs, v_permlane32_swap: wave halves). Every row gets the state
//     entering its run from the carry (the state entering the chunk), and every lane the carry
//     into the next chunk (the total of the 4 runs applied to the carry), kept in a register:
//     the chunk carry never leaves the wave.
//   * Fix pass: each lane re-runs its run's recurrence from the state entering it with the stored
//     dA and input terms (one FMA per step: no exp is recomputed) and forms C h.
//   * dt and dt u of a step come from the lane of its row that computed them, through a DPP row
//     broadcast folded into the multiply (as in the sequential lane-per-state kernel); B and C are
//     staged per chunk in LDS by the workgroup (W channels of one batch) and read with 16-byte
//     LDS reads; the sum over states goes through the wave's own LDS area, in state order.
// With CK the state entering every run, which the combine produces anyway, is the state before a
// 16-step segment: it is stored as the segment's checkpoint (the states saved for the backward).
// Per element: the sequential kernel's 5 operations (2 broadcast multiplies, exp, FMA, C h) plus
// the fix pass's FMA; per chunk and lane the row sum of dt, one exp and about 15 operations of
// combine. It exists for shapes with too few (batch, channel, state) chains to fill the GPU
// sequentially (long sequences of few channels, the L = 100 000 DNA inputs of "Mamba实战…" §4.1):
// a wave per channel instead of a wave per 4 channels.
#pragma once

#include "common.hpp"
#include "scan_ls.hpp"

namespace mscan {

constexpr int kLpK = 16;                     // steps per run (one per lane of a row)
constexpr int kLpT = 4 * kLpK;               // steps per chunk: 4 runs
constexpr int kLpRowP = kLpT + 4;            // LDS floats per staged state row of B or C
constexpr int kLpPRow = 16 * (kLpK + 4) + 16;  // LDS floats per run of the C h transposition

// (a1, b1) then (a2, b2): h -> a2 (a1 h + b1) + b2. Decay products are kept finite (an
// overflowing product would otherwise turn a zero state into NaN where the sequential
// recurrence keeps it zero).
__device__ __forceinline__ float lp_cap(float a) { return __builtin_fminf(a, 3.4028234663852886e38f); }

// ZOH: B discretised by zero-order hold (the input term's coefficient of B from zoh_coef2_f, times
// u, times B), in the local pass where the decays are formed.
template <typename T, int W, bool SOFTPLUS, bool HAS_Z, bool VEC, bool CK, bool ZOH>
__global__ __launch_bounds__(64 * W) void scan_lp_kernel(ScanParams p) {
    __shared__ __align__(16) float s_p[W * 4 * kLpPRow];
    __shared__ __align__(16) float s_bc[2][2][16 * kLpRowP];  // [chunk parity][B|C][state][step]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t blocks = (p.dim + W - 1) / W;
    const int64_t b = blockIdx.x / blocks;
    const int64_t d0 = (blockIdx.x - b * blocks) * W;
    const int r = lane >> 4, n = lane & 15;  // run (row) and state; n is also the lane's step in its run
    const bool valid = d0 + wave < p.dim;
    const int64_t d = valid ? d0 + wave : p.dim - 1;
    const int64_t L = p.len;

    const float an = p.A[d * p.sA_d + n];
    const float a2 = an * kLog2e;
    const float ia = an != 0.0f ? 1.0f / an : 0.0f;  // zero-order hold only
    float carry = p.h0 ? p.h0[b * p.sh0_b + d * p.sh0_d + n] : 0.0f;
    const float bias = p.bias ? p.bias[d * p.sbias] : 0.0f;
    const float Dv = p.D ? p.D[d * p.sD] : 0.0f;  // no skip term: D = 0
    float* const prow = s_p + (wave * 4 + r) * kLpPRow;  // this run's C h block: [state][step]

    // Buffer descriptors with 32-bit byte offsets (the host checks that they fit): one row of
    // u / delta / z / y per wave, one batch of B / C per workgroup; the chunk's offset is an SGPR.
    constexpr uint32_t es = sizeof(T);
    auto row_rsrc = [&](const void* base, int64_t sb, int64_t sd) __attribute__((always_inline)) {
        const T* row0 = static_cast<const T*>(base) + b * sb + d * sd;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(row0), 0, (int)(L * es), kLsWord3);
    };
    const __amdgpu_buffer_rsrc_t ur = row_rsrc(p.u, p.su_b, p.su_d);
    const __amdgpu_buffer_rsrc_t xr = row_rsrc(p.delta, p.sdt_b, p.sdt_d);
    const __amdgpu_buffer_rsrc_t zr = HAS_Z ? row_rsrc(p.z, p.sz_b, p.sz_d) : ur;
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(p.y + b * p.sy_b + d * p.sy_d, 0, (int)(L * 4), kLsWord3);
    const uint32_t st_l = (uint32_t)(r * kLpK + n);  // this lane's step within a chunk
    // saved states (CK): (segment, state) of this channel, segment 4 k + r entered by run r of
    // chunk k; past the last segment the store gets an offset past the range and is dropped
    const __amdgpu_buffer_rsrc_t ckr = __builtin_amdgcn_make_buffer_rsrc(
        CK ? p.ck + (b * p.dim + d) * p.ck_nseg * 16 : p.y, 0, CK ? (int)(p.ck_nseg * 16 * 4) : 0, kLsWord3);
    const uint32_t ock = valid ? (uint32_t)(r * 16 + n) * 4u : kLsDropBase;

    auto load_el = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff) __attribute__((always_inline)) {
        if constexpr (sizeof(T) == 2)
            return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, (int)soff, 0);
        else
            return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, (int)soff, 0);
    };
    auto widen = [](uint32_t v) __attribute__((always_inline)) {
        return __uint_as_float(sizeof(T) == 2 ? v << 16 : v);
    };

    // B / C staging: slots of 4 steps (B|C, state, quarter-step group), SPT per thread, slot =
    // tid + 64 W k; a wave's 64 slots share their B|C half (16 kLpK slots per tensor)
    constexpr int kSlots = 2 * 16 * (kLpT / 4);
    constexpr int SPT = kSlots / (64 * W);
    static_assert(SPT * 64 * W == kSlots && SPT >= 1, "staging slots per thread");
    uint32_t sofs[SPT], sofs_row[SPT];
    float* sdst[SPT];
    __amdgpu_buffer_rsrc_t bcr[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const int slot = tid + 64 * W * k;
        const int q = __builtin_amdgcn_readfirstlane(slot / (kSlots / 2));
        const int s2 = slot % (kSlots / 2);
        const int sn = s2 / (kLpT / 4), st4 = (s2 % (kLpT / 4)) * 4;
        const int64_t sb = q ? p.sC_b : p.sB_b, snn = q ? p.sC_n : p.sB_n;
        bcr[k] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>(static_cast<const void*>(static_cast<const T*>(q ? p.C : p.B) + b * sb)), 0,
            (int)((15 * snn + L) * es), kLsWord3);
        sofs_row[k] = (uint32_t)(sn * snn) * es;
        sofs[k] = sofs_row[k] + st4 * es;
        sdst[k] = &s_bc[0][q][sn * kLpRowP + st4];
    }
    constexpr int kBufStride = 2 * 16 * kLpRowP;
    auto stage_load = [&](int64_t k, bool tail, uint32_t (&v)[SPT][4]) __attribute__((always_inline)) {
        const uint32_t t0 = (uint32_t)(k * kLpT);
        if (!tail) {
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                if constexpr (VEC) {
                    load4_raw<T>(bcr[s], sofs[s], t0 * es, v[s]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[s][i] = load_el(bcr[s], sofs[s] + i * es, t0 * es);
                }
            }
        } else {
            // past len: the row's last value (finite wherever the true result is)
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t t = t0 + (sofs[s] - sofs_row[s]) / es + i;
                    const uint32_t tc = t < (uint32_t)L ? t : (uint32_t)L - 1;
                    v[s][i] = load_el(bcr[s], sofs_row[s] + tc * es, 0);
                }
                if constexpr (VEC && sizeof(T) == 2) pack4_bf16(v[s]);
            }
        }
    };
    auto stage_store = [&](int buf, const uint32_t (&v)[SPT][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < SPT; ++s)
            *reinterpret_cast<float4*>(sdst[s] + buf * kBufStride) = widen4<T, VEC>(v[s]);
    };

    // raw per-(channel, step) inputs of this lane's step of a chunk, one chunk ahead
    struct Raw {
        uint32_t x, u, z;
    };
    constexpr uint32_t kNegInf = sizeof(T) == 2 ? 0xFF80u : 0xFF800000u;
    auto fetch = [&](int64_t k, bool tail, Raw& w) __attribute__((always_inline)) {
        const uint32_t t0 = (uint32_t)(k * kLpT);
        if (!tail) {
            w.x = load_el(xr, st_l * es, t0 * es);
            w.u = load_el(ur, st_l * es, t0 * es);
            w.z = HAS_Z ? load_el(zr, st_l * es, t0 * es) : 0u;
        } else {
            // past len: u and z from the row's last step, delta = -inf so that dt = 0 exactly
            // (softplus and exp both give 0): decay 1, no input, the state is carried unchanged
            const uint32_t t = t0 + st_l;
            const uint32_t tj = t < (uint32_t)L ? t : (uint32_t)L - 1;
            const uint32_t xv = load_el(xr, tj * es, 0);
            w.x = t < (uint32_t)L ? xv : kNegInf;
            w.u = load_el(ur, tj * es, 0);
            w.z = HAS_Z ? load_el(zr, tj * es, 0) : 0u;
        }
    };

    // per-(channel, step) factors of this lane's step: dt, dt u (read by its row through the
    // broadcast), u and the gate for the epilogue
    float dt, dtu, uv, gz;
    auto prologue = [&](const Raw& w) __attribute__((always_inline)) {
        const float xb = widen(w.x) + bias;
        dt = SOFTPLUS ? softplus_f(xb) : hw_exp2(xb * kLog2e);
        uv = widen(w.u);
        dtu = ZOH ? uv : dt * uv;  // u with the zero-order hold, whose coefficient replaces dt
        gz = HAS_Z ? silu_f(widen(w.z)) : 1.0f;
    };

    const int64_t nch = (L + kLpT - 1) / kLpT;
    const bool ragged = L % kLpT != 0;
    {
        Raw w0;
        fetch(0, ragged && nch == 1, w0);
        uint32_t v[SPT][4];
        stage_load(0, ragged && nch == 1, v);
        stage_store(0, v);
        prologue(w0);
    }
    const bool row1 = (r & 1) != 0, row2 = (r & 2) != 0;
    for (int64_t k = 0; k < nch; ++k) {
        const uint32_t t0 = (uint32_t)(k * kLpT);
        const int buf = (int)(k & 1);
        const int64_t kn = k + 1 < nch ? k + 1 : k;
        const bool next_tail = ragged && kn == nch - 1;
        __syncthreads();  // chunk k staged; every wave is done with chunk k-1's buffer
        uint32_t sv[SPT][4];
        stage_load(kn, next_tail, sv);
        Raw nx;
        fetch(kn, next_tail, nx);

        // local pass over this lane's run (state n, steps r K .. r K + K - 1 of the chunk)
        float dA[kLpK], bu[kLpK];
        {
            const float* sb = &s_bc[buf][0][n * kLpRowP + r * kLpK];
            float Bv[kLpK];
#pragma unroll
            for (int q = 0; q < kLpK / 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(sb + 4 * q);
                Bv[4 * q] = v.x, Bv[4 * q + 1] = v.y, Bv[4 * q + 2] = v.z, Bv[4 * q + 3] = v.w;
            }
            float hl = 0.0f;
#define MSCAN_LP_LOCAL(S)                                                                   \
    if constexpr (ZOH) {                                                                    \
        const float dtb = row_bcast<S>(dt), x2 = dtb * a2;                                  \
        dA[S] = hw_exp2(x2);                                                                \
        bu[S] = zoh_coef2_f(dtb, x2, dA[S], ia) * row_bcast<S>(dtu) * Bv[S];                \
    } else {                                                                                \
        dA[S] = hw_exp2(row_bcast<S>(dt) * a2);                                             \
        bu[S] = row_bcast<S>(dtu) * Bv[S];                                                  \
    }                                                                                       \
    hl = (S) == 0 ? bu[S] : __builtin_fmaf(dA[S], hl, bu[S]);
            MSCAN_LP_LOCAL(0) MSCAN_LP_LOCAL(1) MSCAN_LP_LOCAL(2) MSCAN_LP_LOCAL(3)
            MSCAN_LP_LOCAL(4) MSCAN_LP_LOCAL(5) MSCAN_LP_LOCAL(6) MSCAN_LP_LOCAL(7)
            MSCAN_LP_LOCAL(8) MSCAN_LP_LOCAL(9) MSCAN_LP_LOCAL(10) MSCAN_LP_LOCAL(11)
            MSCAN_LP_LOCAL(12) MSCAN_LP_LOCAL(13) MSCAN_LP_LOCAL(14) MSCAN_LP_LOCAL(15)
#undef MSCAN_LP_LOCAL

            // the run's decay product exp(A * sum of its dt): the row's inclusive prefix sum of
            // dt (lane 15 ends with the total), read by the whole row through the broadcast
            float s = dt;
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x111, 0xF, 0xF, false));
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x112, 0xF, 0xF, false));
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x114, 0xF, 0xF, false));
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x118, 0xF, 0xF, false));
            const float ar = lp_cap(hw_exp2(row_bcast<15>(s) * a2));

            // combine the 4 runs' pairs: row pairs, then wave halves
            const auto pa = __builtin_amdgcn_permlane16_swap(__float_as_uint(ar), __float_as_uint(ar), false, false);
            const auto pb = __builtin_amdgcn_permlane16_swap(__float_as_uint(hl), __float_as_uint(hl), false, false);
            const float loA = __uint_as_float(pa[0]), hiA = __uint_as_float(pa[1]);  // runs 2i, 2i+1
            const float lob = __uint_as_float(pb[0]), hib = __uint_as_float(pb[1]);
            const float qA = lp_cap(loA * hiA), qb = __builtin_fmaf(hiA, lob, hib);  // runs 2i then 2i+1
            const auto sa = __builtin_amdgcn_permlane32_swap(__float_as_uint(qA), __float_as_uint(qA), false, false);
            const auto sbb = __builtin_amdgcn_permlane32_swap(__float_as_uint(qb), __float_as_uint(qb), false, false);
            const float LA = __uint_as_float(sa[0]), HA = __uint_as_float(sa[1]);  // runs 0-1, runs 2-3
            const float Lb = __uint_as_float(sbb[0]), Hb = __uint_as_float(sbb[1]);
            // the state entering run r: runs 0 .. r-1 applied to the carry
            const float h1 = row2 ? __builtin_fmaf(LA, carry, Lb) : carry;
            const float hin = row1 ? __builtin_fmaf(loA, h1, lob) : h1;
            if constexpr (CK)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hin), ckr, (int)ock, (int)(t0 * 4u), 0);
            // the carry into the next chunk: all 4 runs applied to it
            const float tA = lp_cap(LA * HA), tb = __builtin_fmaf(HA, Lb, Hb);
            carry = __builtin_fmaf(tA, carry, tb);

            // fix pass: the run again from its entering state, C h into the run's LDS block
            const float* sc = &s_bc[buf][1][n * kLpRowP + r * kLpK];
            float* const sp = prow + n * (kLpK + 4);
            float h = hin;
#pragma unroll
            for (int q = 0; q < kLpK / 4; ++q) {
                const float4 c = *reinterpret_cast<const float4*>(sc + 4 * q);
                float4 o;
                h = __builtin_fmaf(dA[4 * q], h, bu[4 * q]);
                o.x = c.x * h;
                h = __builtin_fmaf(dA[4 * q + 1], h, bu[4 * q + 1]);
                o.y = c.y * h;
                h = __builtin_fmaf(dA[4 * q + 2], h, bu[4 * q + 2]);
                o.z = c.z * h;
                h = __builtin_fmaf(dA[4 * q + 3], h, bu[4 * q + 3]);
                o.w = c.w * h;
                *reinterpret_cast<float4*>(sp + 4 * q) = o;
            }
        }
        // the next chunk's B / C into the other buffer (its last readers passed the barrier above)
        stage_store(buf ^ 1, sv);
        const float u0 = uv, g0 = gz;
        prologue(nx);
        __builtin_amdgcn_wave_barrier();
        // run r, step n: the sum over the 16 states' C h terms, in state order
        float yv = prow[n];
#pragma unroll
        for (int m = 1; m < 16; ++m) yv += prow[m * (kLpK + 4) + n];
        __builtin_amdgcn_wave_barrier();
        const float o = __builtin_fmaf(Dv, u0, yv) * g0;
        const uint32_t t = t0 + st_l;
        const uint32_t oy = (valid && t < (uint32_t)L) ? st_l * 4u : kLsDropBase;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), yr, (int)oy, (int)(t0 * 4u), 0);
    }
    if (p.last_state && valid && r == 0) p.last_state[b * p.sls_b + d * p.sls_d + n] = carry;
}

// ---------------------------------------------------------------------------------------------
// host side

constexpr int kLpW = 4;  // channels (waves) per workgroup

// 16 states (either input term; the zero-order hold without saved states, which only the Euler
// backward reads), and byte offsets within a row (u, delta, z, y), within a batch's B / C and
// within a channel's saved states that fit 31 bits.
inline bool lp_eligible(const ScanParams& q, int64_t es) {
    if (q.dstate != 16 || (q.zoh_b && q.ck)) return false;
    const int64_t lim = (int64_t)1 << 31;
    if (q.len * 4 >= lim) return false;
    if (q.ck && q.ck_nseg * 16 * 4 >= lim) return false;
    if ((15 * q.sB_n + q.len) * es >= lim || (15 * q.sC_n + q.len) * es >= lim) return false;
    if (q.batch * ((q.dim + kLpW - 1) / kLpW) > 0x7fffffff) return false;
    return true;
}

template <typename T, bool SP, bool HZ, bool VEC>
int launch_lp_cfg(const ScanParams& q, hipStream_t stream) {
    void* args[] = {const_cast<ScanParams*>(&q)};
    const int64_t groups = q.batch * ((q.dim + kLpW - 1) / kLpW);
    // saving the segment states is a separate instantiation: the plain forward issues no stores
    // for it; so is the zero-order hold (never with saved states)
    const void* fn = q.zoh_b ? reinterpret_cast<const void*>(&scan_lp_kernel<T, kLpW, SP, HZ, VEC, false, true>)
                     : q.ck  ? reinterpret_cast<const void*>(&scan_lp_kernel<T, kLpW, SP, HZ, VEC, true, false>)
                             : reinterpret_cast<const void*>(&scan_lp_kernel<T, kLpW, SP, HZ, VEC, false, false>);
    return hipLaunchKernel(fn, dim3((unsigned)groups), dim3(64 * kLpW), args, 0, stream) == hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

template <typename T, bool SP, bool HZ>
int launch_lp_vec(const ScanParams& q, hipStream_t stream) {
    const auto al = [](const void* ptr, int64_t sb, int64_t sn) {
        return reinterpret_cast<uintptr_t>(ptr) % (4 * sizeof(T)) == 0 && sb % 4 == 0 && sn % 4 == 0;
    };
    if (al(q.B, q.sB_b, q.sB_n) && al(q.C, q.sC_b, q.sC_n)) return launch_lp_cfg<T, SP, HZ, true>(q, stream);
    return launch_lp_cfg<T, SP, HZ, false>(q, stream);
}

template <typename T>
int launch_lp(const ScanParams& q, hipStream_t stream) {
    if (!lp_eligible(q, sizeof(T))) return MAMBA_SCAN_ERR_UNSUPPORTED;
    const bool sp = q.softplus != 0, hz = q.z != nullptr;
    if (sp && hz) return launch_lp_vec<T, true, true>(q, stream);
    if (sp) return launch_lp_vec<T, true, false>(q, stream);
    if (hz) return launch_lp_vec<T, false, true>(q, stream);
    return launch_lp_vec<T, false, false>(q, stream);
}

}  // namespace mscan
