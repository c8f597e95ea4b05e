// Lane-per-state forward kernel for 16 states (gfx950).
//
// Computes the same operation as the tiled kernel (the recurrence of "Mamba代码实战…" §3.1-§3.3
// and §6, the output contraction of "Mamba-minimal项目解析…" 关键技术点 1, the optional initial
// state of "手把手用PyTorch实现Mamba的SSM层…" §3.1), decomposed the other way round: one lane per
// (channel, state), a wave = 4 channels x 16 states (lane 16c + n: channel c, state n).
//   * The sum over states of an output is a wave's own business: each lane writes its C h terms
//     to the wave's LDS area and, per 32-step chunk, sums the 16 states' terms of 2 outputs. No
//     partial sums cross waves.
//   * dt and dt*u of a (channel, step) are computed once, by one lane of the channel's 16-lane
//     row, and reach the other 15 lanes through a DPP row broadcast folded into the multiply that
//     consumes them (v_mul_f32_dpp ... row_newbcast), at no instruction cost.
//   * B and C vary along the lanes (one state each) but not along the channels: a workgroup (4
//     waves, 16 channels of one batch) stages each 32-step chunk of them in LDS as fp32, one
//     chunk ahead (the workgroup's only barrier, one per chunk), and every lane reads its
//     state's values with 16-byte LDS reads that the 4 rows of a wave share (per-lane vector
//     loads from memory, 4 times duplicated, ran the kernel at half speed).
//   * The grid is batch x dim / 16 workgroups of 4 waves: at the Mamba-130m shape 3072 waves,
//     3 per SIMD on every CU (the 64-channel tiling leaves a quarter of the CUs idle there).
// Per step a lane does v_mul (dt A log2e, broadcast dt), v_exp, v_mul (dt u B, broadcast dt u),
// v_fma (h) and v_mul (C h); every 4 steps one 16-byte LDS write of the four C h terms. Per
// 32-step chunk each lane then sums the 16 states' terms of 2 (channel, step) outputs from LDS and
// finishes them (skip, gate, store), after having computed dt / dt u / gate for those 2 steps of
// the next chunk. The issue slots are the bound: about 94 % of every SIMD's cycles issue VALU.
#pragma once

#include "common.hpp"

namespace mscan {

constexpr int kLsWaves = 4;                  // waves per workgroup
constexpr int kLsT = 32;                     // steps per chunk
constexpr int kLsH = 16;                     // steps per B/C half-chunk
constexpr int kLsRowP = kLsT + 4;            // LDS floats per state row of one channel
constexpr int kLsChanP = 16 * kLsRowP + 32;  // LDS floats per channel (rows 0..15 + bank skew)
constexpr uint32_t kLsWord3 = 0x00020000u;   // buffer descriptor word 3: raw 32-bit dwords
constexpr uint32_t kLsDropBase = 0x80000000u; // byte offset past any range: store dropped

template <int LANE>
__device__ __forceinline__ float row_bcast(float x) {
    // every lane of each 16-lane row reads lane LANE of that row (bound_ctrl: all lanes valid)
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + LANE, 0xF, 0xF, true));
}

template <int V>
struct LsIdx {
    static constexpr int value = V;
};

// f(LsIdx<I>{}) for I = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void bl_for_ls(F&& f) {
    if constexpr (B < E) {
        f(LsIdx<B>{});
        bl_for_ls<B + 1, E>(f);
    }
}

struct LsRegs {
    float h, a2, ia;  // ia = 1 / A (zero-order hold only)
    float dt[2], dtu[2];  // dtu: dt u, or u with the zero-order hold
    float Bv[2][kLsH], Cv[2][kLsH];  // [half][step] of this lane's state rows of B and C
    float pv[4];
    float* sp;  // this lane's state row in LDS
};

// Steps S .. kLsH-1 of half-chunk HALF (buffer BUF) of the recurrence. The input term: dt u B
// (Euler), or with the zero-order hold (ZOH) its coefficient of B times u, times B.
template <int HALF, int BUF, int S, bool ZOH>
__device__ __forceinline__ void ls_steps(LsRegs& r) {
    if constexpr (S < kLsH) {
        constexpr int s = HALF * kLsH + S;  // step within the chunk
        if constexpr (ZOH) {
            const float dtb = row_bcast<s / 2>(r.dt[s % 2]);
            const float x2 = dtb * r.a2;
            const float dA = hw_exp2(x2);
            const float inc = zoh_coef2_f(dtb, x2, dA, r.ia) * row_bcast<s / 2>(r.dtu[s % 2]) * r.Bv[BUF][S];
            r.h = __builtin_fmaf(dA, r.h, inc);
        } else {
            const float dA = hw_exp2(row_bcast<s / 2>(r.dt[s % 2]) * r.a2);
            r.h = __builtin_fmaf(dA, r.h, row_bcast<s / 2>(r.dtu[s % 2]) * r.Bv[BUF][S]);
        }
        r.pv[s % 4] = r.Cv[BUF][S] * r.h;
        if constexpr (s % 4 == 3)
            *reinterpret_cast<float4*>(r.sp + (s - 3)) = float4{r.pv[0], r.pv[1], r.pv[2], r.pv[3]};
        ls_steps<HALF, BUF, S + 1, ZOH>(r);
    }
}

// Staged values of 4 consecutive steps of B or C, as raw bits. PACKED (bf16 rows staged with
// vector loads): v[0], v[1] hold the 4 values as two bf16 pairs; otherwise one value per entry.
// The bits are only unpacked / widened where they are written to LDS: an ALU operation next to
// the load would make the compiler wait for the load there.
template <typename T>
__device__ __forceinline__ void load4_raw(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff, uint32_t (&v)[4]) {
    // one 8-byte (bf16) or 16-byte (fp32) buffer load; the caller guarantees 4-element alignment
    if constexpr (sizeof(T) == 2) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, (int)soff, 0);
        v[0] = w[0], v[1] = w[1], v[2] = 0u, v[3] = 0u;
    } else {
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, (int)soff, 0);
        v[0] = w[0], v[1] = w[1], v[2] = w[2], v[3] = w[3];
    }
}

template <typename T, bool PACKED>
__device__ __forceinline__ float4 widen4(const uint32_t (&v)[4]) {
    if constexpr (sizeof(T) == 2 && PACKED)
        return float4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u), __uint_as_float(v[1] << 16),
                      __uint_as_float(v[1] & 0xFFFF0000u)};
    else if constexpr (sizeof(T) == 2)
        return float4{__uint_as_float(v[0] << 16), __uint_as_float(v[1] << 16), __uint_as_float(v[2] << 16),
                      __uint_as_float(v[3] << 16)};
    else
        return float4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
}

// element bits e0..e3 (bf16 zero-extended) into the PACKED layout
__device__ __forceinline__ void pack4_bf16(uint32_t (&v)[4]) {
    v[0] = v[0] | (v[1] << 16), v[1] = v[2] | (v[3] << 16), v[2] = 0u, v[3] = 0u;
}

// VEC: B and C rows 4-element aligned, staged with one vector load per 4 steps; ZOH: B
// discretised by zero-order hold
template <typename T, bool SOFTPLUS, bool HAS_Z, bool VEC, bool CK, bool ZOH>
__global__ __launch_bounds__(64 * kLsWaves) __attribute__((amdgpu_waves_per_eu(3)))
void scan_ls_kernel(ScanParams p) {
    __shared__ __align__(16) float s_p[kLsWaves * 4 * kLsChanP];
    __shared__ __align__(16) float s_bc[2][2][16 * kLsRowP];  // [chunk parity][B|C][state][step]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t blocks = (p.dim + 15) / 16;
    const int64_t b = blockIdx.x / blocks;
    const int64_t d0 = (blockIdx.x - b * blocks) * 16 + wave * 4;
    const int c = lane >> 4, n = lane & 15;
    const bool valid = d0 + c < p.dim;
    const int64_t d = valid ? d0 + c : p.dim - 1;
    const int64_t L = p.len;

    LsRegs r;
    {
        const float an = p.A[d * p.sA_d + n];
        r.a2 = an * kLog2e;
        r.ia = an != 0.0f ? 1.0f / an : 0.0f;
    }
    r.h = p.h0 ? p.h0[b * p.sh0_b + d * p.sh0_d + n] : 0.0f;
    const float bias = p.bias ? p.bias[d * p.sbias] : 0.0f;
    const float Dv = p.D ? p.D[d * p.sD] : 0.0f;  // no skip term: D = 0
    float* const chan = s_p + (wave * 4 + c) * kLsChanP;
    r.sp = chan + n * kLsRowP;

    // All global accesses go through buffer descriptors with 32-bit byte offsets (the host checks
    // that they fit): a descriptor per wave for its 4 rows of u / delta / z / y, one per batch for
    // B / C. Offsets advance by one chunk per iteration; in a chunk that reaches past len the
    // step index is clamped to len - 1 (loads) or the store gets an offset past the range.
    constexpr uint32_t es = sizeof(T);
    const int64_t d0c = d0 < p.dim ? d0 : p.dim - 1;           // first row of the wave, clamped
    const int64_t dl = d0 + 3 < p.dim ? d0 + 3 : p.dim - 1;   // last row of the wave, clamped
    const uint32_t dr = (uint32_t)(d - d0c);                  // this lane's row in the wave
    auto rows_rsrc = [&](const void* base, int64_t sb, int64_t sd) __attribute__((always_inline)) {
        const T* row0 = static_cast<const T*>(base) + b * sb + d0c * sd;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(row0), 0, (int)(((dl - d0c) * sd + L) * es), kLsWord3);
    };
    const __amdgpu_buffer_rsrc_t ur = rows_rsrc(p.u, p.su_b, p.su_d);
    const __amdgpu_buffer_rsrc_t xr = rows_rsrc(p.delta, p.sdt_b, p.sdt_d);
    const __amdgpu_buffer_rsrc_t zr = HAS_Z ? rows_rsrc(p.z, p.sz_b, p.sz_d) : ur;
    const uint32_t ou = dr * (uint32_t)p.su_d * es, ox = dr * (uint32_t)p.sdt_d * es;
    const uint32_t oz = HAS_Z ? dr * (uint32_t)p.sz_d * es : 0u;
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        p.y + b * p.sy_b + d0c * p.sy_d, 0, (int)(((dl - d0c) * p.sy_d + L) * 4), kLsWord3);
    const uint32_t oy_l = valid ? (dr * (uint32_t)p.sy_d + 2 * n) * 4u : kLsDropBase;
    // saved states (CK): the state before every 16-step segment, (row, segment, state) from the
    // wave's first row, stored at the end of each chunk beside y
    const __amdgpu_buffer_rsrc_t ckr = __builtin_amdgcn_make_buffer_rsrc(
        CK ? p.ck + (b * p.dim + d0c) * p.ck_nseg * 16 : p.y, 0,
        CK ? (int)((dl - d0c + 1) * p.ck_nseg * 16 * 4) : 0, kLsWord3);
    const uint32_t ock = valid ? (dr * (uint32_t)p.ck_nseg * 16 + n) * 4u : kLsDropBase;

    // raw bits of one element; widened to fp32 (widen) only where the value is used, so that a
    // load inside a branch is not waited for inside it
    // soff: the chunk's byte offset, wave-uniform (an SGPR), so that advancing a chunk costs no
    // vector instruction
    auto load_el = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff) __attribute__((always_inline)) {
        if constexpr (sizeof(T) == 2)
            return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, (int)soff, 0);
        else
            return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, (int)soff, 0);
    };
    auto widen = [](uint32_t v) __attribute__((always_inline)) {
        return __uint_as_float(sizeof(T) == 2 ? v << 16 : v);
    };

    // B / C staging role: thread -> (B|C, state, 4 steps of the chunk); B by waves 0-1, C by 2-3
    const int sq = wave >> 1, sn = (wave & 1) * 8 + (lane >> 3), st4 = (lane & 7) * 4;  // sq wave-uniform
    const __amdgpu_buffer_rsrc_t bcr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const T*>(sq ? p.C : p.B) + b * (sq ? p.sC_b : p.sB_b))), 0,
        (int)((15 * (sq ? p.sC_n : p.sB_n) + L) * es), kLsWord3);
    const uint32_t obc = (uint32_t)(sn * (sq ? p.sC_n : p.sB_n)) * es;
    float* const sdst = &s_bc[0][sq][sn * kLsRowP + st4];
    constexpr int kBufStride = 2 * 16 * kLsRowP;
    const uint32_t obc_l = obc + st4 * es;
    auto stage_load = [&](int64_t k, bool tail, uint32_t (&v)[4]) __attribute__((always_inline)) {
        const uint32_t t0 = (uint32_t)(k * kLsT);
        if (!tail) {
            if constexpr (VEC) {
                load4_raw<T>(bcr, obc_l, t0 * es, v);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = load_el(bcr, obc_l + j * es, t0 * es);
            }
        } else {
            // past len: the row's last value (finite wherever the true result is)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t tj = t0 + st4 + j < (uint32_t)L ? t0 + st4 + j : (uint32_t)L - 1;
                v[j] = load_el(bcr, obc + tj * es, 0);
            }
            if constexpr (VEC && sizeof(T) == 2) pack4_bf16(v);
        }
    };

    // raw per-(channel, step) inputs of this lane's two steps 2n, 2n+1 of a chunk, one chunk ahead
    struct Raw {
        uint32_t x[2], u[2], z[2];
    };
    const uint32_t ou_l = ou + 2 * n * es, ox_l = ox + 2 * n * es, oz_l = oz + 2 * n * es;
    constexpr uint32_t kNegInf = sizeof(T) == 2 ? 0xFF80u : 0xFF800000u;
    auto fetch = [&](int64_t k, bool tail, Raw& w) __attribute__((always_inline)) {
        const uint32_t t0 = (uint32_t)(k * kLsT);
        if (!tail) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                w.x[j] = load_el(xr, ox_l + j * es, t0 * es);
                w.u[j] = load_el(ur, ou_l + j * es, t0 * es);
                w.z[j] = HAS_Z ? load_el(zr, oz_l + j * es, t0 * es) : 0u;
            }
        } else {
            // past len: u and z from the row's last step, delta = -inf so that dt = 0 (softplus
            // and exp both give exactly 0): decay 1, no input, the state is carried unchanged
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t t = t0 + 2 * n + j;
                const uint32_t tj = t < (uint32_t)L ? t : (uint32_t)L - 1;
                const uint32_t xv = load_el(xr, ox + tj * es, 0);
                w.x[j] = t < (uint32_t)L ? xv : kNegInf;
                w.u[j] = load_el(ur, ou + tj * es, 0);
                w.z[j] = HAS_Z ? load_el(zr, oz + tj * es, 0) : 0u;
            }
        }
    };
    // this lane's state rows of B and C for half-chunk `half` of the staged chunk `buf`
    auto read_bc = [&](int buf, int half) __attribute__((always_inline)) {
        const float* sb = &s_bc[buf][0][n * kLsRowP + half * kLsH];
        const float* sc = &s_bc[buf][1][n * kLsRowP + half * kLsH];
#pragma unroll
        for (int q = 0; q < kLsH / 4; ++q) {
            const float4 vb = *reinterpret_cast<const float4*>(sb + 4 * q);
            const float4 vc = *reinterpret_cast<const float4*>(sc + 4 * q);
            float* B = half ? r.Bv[1] : r.Bv[0];
            float* C = half ? r.Cv[1] : r.Cv[0];
            B[4 * q] = vb.x, B[4 * q + 1] = vb.y, B[4 * q + 2] = vb.z, B[4 * q + 3] = vb.w;
            C[4 * q] = vc.x, C[4 * q + 1] = vc.y, C[4 * q + 2] = vc.z, C[4 * q + 3] = vc.w;
        }
    };

    // Per-(channel, step) factors of this lane's two steps of chunk k: dt and dt*u (u with the
    // zero-order hold; read by the whole row through the broadcast), and u and the gate for the
    // epilogue.
    float uv[2], gz[2];
    auto prologue = [&](const Raw& w) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float xb = widen(w.x[j]) + bias;
            r.dt[j] = SOFTPLUS ? softplus_f(xb) : hw_exp2(xb * kLog2e);
            uv[j] = widen(w.u[j]);
            r.dtu[j] = ZOH ? uv[j] : r.dt[j] * uv[j];
            gz[j] = HAS_Z ? silu_f(widen(w.z[j])) : 1.0f;
        }
    };

    // Software pipeline: chunk k+1's raw inputs and B / C are loaded at the top of chunk k and
    // consumed at its end, before chunk k's y stores. The loop head then has no load to wait
    // for, and no wait ever covers a store issued less than a chunk earlier (with loads and
    // stores both in flight, a wait on the vector-memory counter must drain it to zero).
    const int64_t nch = (L + kLsT - 1) / kLsT;
    const bool ragged = L % kLsT != 0;  // the last chunk reaches past len
    {
        Raw w0;
        fetch(0, ragged && nch == 1, w0);
        uint32_t v[4];
        stage_load(0, ragged && nch == 1, v);
        *reinterpret_cast<float4*>(sdst) = widen4<T, VEC>(v);
        prologue(w0);
    }
    for (int64_t k = 0; k < nch; ++k) {
        const uint32_t t0 = (uint32_t)(k * kLsT);
        const int buf = (int)(k & 1);
        const int64_t kn = k + 1 < nch ? k + 1 : k;
        const bool next_tail = ragged && kn == nch - 1;
        __syncthreads();  // chunk k staged; every wave is done with chunk k-1's buffer
        uint32_t sv[4];
        stage_load(kn, next_tail, sv);
        Raw nx;
        fetch(kn, next_tail, nx);
        read_bc(buf, 0);
        read_bc(buf, 1);
        // the states before steps t0 and t0 + 16 (segments 2k and 2k + 1), stored with y
        const float hk0 = r.h;
        ls_steps<0, 0, 0, ZOH>(r);
        const float hk1 = r.h;
        ls_steps<1, 1, 0, ZOH>(r);
        // the next chunk's B / C into the other buffer (its last readers passed the barrier above)
        *reinterpret_cast<float4*>(sdst + (buf ^ 1) * kBufStride) =
            widen4<T, VEC>(sv);
        const float u0 = uv[0], u1 = uv[1], g0 = gz[0], g1 = gz[1];
        prologue(nx);
        __builtin_amdgcn_wave_barrier();
        // channel c, steps 2n and 2n+1: the sum over the 16 states' C h terms, in state order
        float y0, y1;
        {
            const float2 v = *reinterpret_cast<const float2*>(chan + 2 * n);
            y0 = v.x;
            y1 = v.y;
        }
#pragma unroll
        for (int m = 1; m < 16; ++m) {
            const float2 v = *reinterpret_cast<const float2*>(chan + m * kLsRowP + 2 * n);
            y0 += v.x;
            y1 += v.y;
        }
        __builtin_amdgcn_wave_barrier();
        const float o0 = __builtin_fmaf(Dv, u0, y0) * g0, o1 = __builtin_fmaf(Dv, u1, y1) * g1;
        if (!(ragged && k == nch - 1)) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o0), yr, (int)oy_l, (int)(t0 * 4u), 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o1), yr, (int)(oy_l + 4u), (int)(t0 * 4u), 0);
        } else {
            const uint32_t t = t0 + 2 * n;
            const uint32_t a0 = t < (uint32_t)L ? oy_l : kLsDropBase;
            const uint32_t a1 = t + 1 < (uint32_t)L ? oy_l + 4u : kLsDropBase;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o0), yr, (int)a0, (int)(t0 * 4u), 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o1), yr, (int)a1, (int)(t0 * 4u), 0);
        }
        if constexpr (CK) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hk0), ckr, (int)ock, (int)(t0 * 4u), 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hk1), ckr,
                                                  (int)(t0 + kLsH < (uint32_t)L ? ock + 64u : kLsDropBase),
                                                  (int)(t0 * 4u), 0);
        }
    }
    if (p.last_state && valid) p.last_state[b * p.sls_b + d * p.sls_d + n] = r.h;
}

// ---------------------------------------------------------------------------------------------
// 32 and 64 states: S = N / 16 states per lane, so that a channel still fills one 16-lane row.
//   * A wave = 4 channels (rows), as at 16 states; lane j of a row holds states j, j + 16, ...,
//     j + 16 (S - 1) of its channel, in chunks of 16 steps.
//   * Lane j computes the per-(channel, step) factors of step j of the chunk; the row reads them
//     through one DPP row broadcast per factor and step, which then serves the lane's S states.
//   * Per step a lane adds its S states' C h terms (in state order) and writes one value per step
//     to the wave's LDS area; lane j then sums step j over the row's 16 lanes, in lane order, and
//     finishes and stores y. The sum over states is thus taken in the order: states n, n + 16, ..
//     within a lane, then lanes 0 .. 15.
//   * B / C: the workgroup (4 waves, 16 channels of one batch) stages N states x 16 steps of each
//     per chunk in LDS, one chunk ahead; a lane reads its states' rows 4 steps at a time.
constexpr int kLwT = 16;                      // steps per chunk
constexpr int kLwRowP = kLwT + 4;             // LDS floats per lane row of C h sums
constexpr int kLwChanP = 16 * kLwRowP + 16;   // one channel's 16 lane rows, skewed by 16 banks

// Staged B / C: unpadded rows of 16 steps (so that 4 workgroups fit a CU at 64 states), the 4-step
// group g of state row m at group (g ^ (m / 4)) % 4: a lane's 16-byte read of one group of its
// state rows, and a staging thread's 16-byte write, touch distinct banks across 16 lanes.
__device__ __forceinline__ int lw_bc_at(int m, int g) { return m * kLwT + (((g ^ (m >> 2)) & 3) << 2); }

template <typename T, int N, bool SOFTPLUS, bool HAS_Z, bool VEC, bool CK, bool ZOH>
__global__ __launch_bounds__(64 * kLsWaves) __attribute__((amdgpu_waves_per_eu(4)))
void scan_ls_wide_kernel(ScanParams p) {
    static_assert(N == 32 || N == 64, "wide lane-per-state kernel: 32 or 64 states");
    constexpr int S = N / 16;          // states per lane
    constexpr int CG = kLsWaves * 4;   // channels per workgroup
    __shared__ __align__(16) float s_p[kLsWaves * 4 * kLwChanP];
    __shared__ __align__(16) float s_bc[2][2][N * kLwT];  // [chunk parity][B|C][state][step], swizzled

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t blocks = (p.dim + CG - 1) / CG;
    const int64_t b = blockIdx.x / blocks;
    const int64_t d0 = (blockIdx.x - b * blocks) * CG + wave * 4;
    const int c = lane >> 4, j = lane & 15;
    const bool valid = d0 + c < p.dim;
    const int64_t d = valid ? d0 + c : p.dim - 1;
    const int64_t L = p.len;

    float h[S], a2[S], ia[S];  // ia = 1 / A (zero-order hold only)
#pragma unroll
    for (int k = 0; k < S; ++k) {
        const float an = p.A[d * p.sA_d + j + 16 * k];
        a2[k] = an * kLog2e;
        ia[k] = an != 0.0f ? 1.0f / an : 0.0f;
        h[k] = p.h0 ? p.h0[b * p.sh0_b + d * p.sh0_d + j + 16 * k] : 0.0f;
    }
    const float bias = p.bias ? p.bias[d * p.sbias] : 0.0f;
    const float Dv = p.D ? p.D[d * p.sD] : 0.0f;  // no skip term: D = 0
    float* const chan = s_p + (wave * 4 + c) * kLwChanP;
    float* const sp = chan + j * kLwRowP;  // this lane's row of C h sums

    constexpr uint32_t es = sizeof(T);
    const int64_t d0c = d0 < p.dim ? d0 : p.dim - 1;
    const int64_t dl = d0 + 3 < p.dim ? d0 + 3 : p.dim - 1;
    const uint32_t dr = (uint32_t)(d - d0c);
    auto rows_rsrc = [&](const void* base, int64_t sb, int64_t sd) __attribute__((always_inline)) {
        const T* row0 = static_cast<const T*>(base) + b * sb + d0c * sd;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(row0), 0, (int)(((dl - d0c) * sd + L) * es), kLsWord3);
    };
    const __amdgpu_buffer_rsrc_t ur = rows_rsrc(p.u, p.su_b, p.su_d);
    const __amdgpu_buffer_rsrc_t xr = rows_rsrc(p.delta, p.sdt_b, p.sdt_d);
    const __amdgpu_buffer_rsrc_t zr = HAS_Z ? rows_rsrc(p.z, p.sz_b, p.sz_d) : ur;
    const uint32_t ou = dr * (uint32_t)p.su_d * es, ox = dr * (uint32_t)p.sdt_d * es;
    const uint32_t oz = HAS_Z ? dr * (uint32_t)p.sz_d * es : 0u;
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        p.y + b * p.sy_b + d0c * p.sy_d, 0, (int)(((dl - d0c) * p.sy_d + L) * 4), kLsWord3);
    const uint32_t oy_l = valid ? (dr * (uint32_t)p.sy_d + j) * 4u : kLsDropBase;
    // saved states (CK): the state before every 16-step segment, one segment per chunk
    const __amdgpu_buffer_rsrc_t ckr = __builtin_amdgcn_make_buffer_rsrc(
        CK ? p.ck + (b * p.dim + d0c) * p.ck_nseg * N : p.y, 0,
        CK ? (int)((dl - d0c + 1) * p.ck_nseg * N * 4) : 0, kLsWord3);
    const uint32_t ock = valid ? (dr * (uint32_t)p.ck_nseg * N + j) * 4u : kLsDropBase;

    auto load_el = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff) __attribute__((always_inline)) {
        if constexpr (sizeof(T) == 2)
            return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, (int)soff, 0);
        else
            return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, (int)soff, 0);
    };
    auto widen = [](uint32_t v) __attribute__((always_inline)) {
        return __uint_as_float(sizeof(T) == 2 ? v << 16 : v);
    };

    // B / C staging: 8 N slots of 4 steps, (B|C, state, quarter of the chunk); N / 32 slots per
    // thread, slot = tid + 256 k, whose B|C half is wave-uniform
    constexpr int SPT = N / 32;
    uint32_t sofs[SPT], sofs_row[SPT];
    float* sdst[SPT];
    __amdgpu_buffer_rsrc_t bcr[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const int slot = wave * 64 + lane + 256 * k;
        const int q = __builtin_amdgcn_readfirstlane(slot / (4 * N));
        const int sn = (slot / 4) % N, st4 = (slot % 4) * 4;
        const int64_t sb = q ? p.sC_b : p.sB_b, snn = q ? p.sC_n : p.sB_n;
        bcr[k] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>(static_cast<const void*>(static_cast<const T*>(q ? p.C : p.B) + b * sb)), 0,
            (int)(((N - 1) * snn + L) * es), kLsWord3);
        sofs_row[k] = (uint32_t)(sn * snn) * es;
        sofs[k] = sofs_row[k] + st4 * es;
        sdst[k] = &s_bc[0][q][lw_bc_at(sn, st4 / 4)];
    }
    constexpr int kBufStride = 2 * N * kLwT;
    auto stage_load = [&](int64_t k, bool tail, uint32_t (&v)[SPT][4]) __attribute__((always_inline)) {
        const uint32_t t0 = (uint32_t)(k * kLwT);
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
            for (int s = 0; s < SPT; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t t = t0 + (sofs[s] - sofs_row[s]) / es + i;
                    const uint32_t tc = t < (uint32_t)L ? t : (uint32_t)L - 1;
                    v[s][i] = load_el(bcr[s], sofs_row[s] + tc * es, 0);
                }
            if constexpr (VEC && sizeof(T) == 2)
#pragma unroll
                for (int s = 0; s < SPT; ++s) pack4_bf16(v[s]);
        }
    };
    auto stage_store = [&](int buf, const uint32_t (&v)[SPT][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < SPT; ++s)
            *reinterpret_cast<float4*>(sdst[s] + buf * kBufStride) = widen4<T, VEC>(v[s]);
    };

    // raw per-(channel, step) inputs of this lane's step j of a chunk, one chunk ahead
    struct Raw {
        uint32_t x, u, z;
    };
    const uint32_t ou_l = ou + j * es, ox_l = ox + j * es, oz_l = oz + j * es;
    constexpr uint32_t kNegInf = sizeof(T) == 2 ? 0xFF80u : 0xFF800000u;
    auto fetch = [&](int64_t k, bool tail, Raw& w) __attribute__((always_inline)) {
        const uint32_t t0 = (uint32_t)(k * kLwT);
        if (!tail) {
            w.x = load_el(xr, ox_l, t0 * es);
            w.u = load_el(ur, ou_l, t0 * es);
            w.z = HAS_Z ? load_el(zr, oz_l, t0 * es) : 0u;
        } else {
            // past len: u and z from the row's last step, delta = -inf so that dt = 0 exactly
            const uint32_t t = t0 + j;
            const uint32_t tj = t < (uint32_t)L ? t : (uint32_t)L - 1;
            const uint32_t xv = load_el(xr, ox + tj * es, 0);
            w.x = t < (uint32_t)L ? xv : kNegInf;
            w.u = load_el(ur, ou + tj * es, 0);
            w.z = HAS_Z ? load_el(zr, oz + tj * es, 0) : 0u;
        }
    };
    float dt, dtu, uv, gz;
    auto prologue = [&](const Raw& w) __attribute__((always_inline)) {
        const float xb = widen(w.x) + bias;
        dt = SOFTPLUS ? softplus_f(xb) : hw_exp2(xb * kLog2e);
        uv = widen(w.u);
        dtu = ZOH ? uv : dt * uv;  // u with the zero-order hold, whose coefficient replaces dt
        gz = HAS_Z ? silu_f(widen(w.z)) : 1.0f;
    };

    // 4 steps Q*4 .. Q*4+3 of the chunk: the lane's S states from B / C staged in buffer buf
    auto steps4 = [&](int buf, auto qc) __attribute__((always_inline)) {
        constexpr int Q = decltype(qc)::value;
        float4 bv[S], cv[S];
#pragma unroll
        for (int k = 0; k < S; ++k) {
            bv[k] = *reinterpret_cast<const float4*>(&s_bc[buf][0][lw_bc_at(j + 16 * k, Q)]);
            cv[k] = *reinterpret_cast<const float4*>(&s_bc[buf][1][lw_bc_at(j + 16 * k, Q)]);
        }
        float pv[4];
        bl_for_ls<0, 4>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            constexpr int st = 4 * Q + i;
            const float dtb = row_bcast<st>(dt), dtub = row_bcast<st>(dtu);
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < S; ++k) {
                const float bb = i == 0 ? bv[k].x : i == 1 ? bv[k].y : i == 2 ? bv[k].z : bv[k].w;
                const float cc = i == 0 ? cv[k].x : i == 1 ? cv[k].y : i == 2 ? cv[k].z : cv[k].w;
                if constexpr (ZOH) {
                    const float x2 = dtb * a2[k];
                    const float dA = hw_exp2(x2);
                    h[k] = __builtin_fmaf(dA, h[k], zoh_coef2_f(dtb, x2, dA, ia[k]) * dtub * bb);
                } else {
                    h[k] = __builtin_fmaf(hw_exp2(dtb * a2[k]), h[k], dtub * bb);
                }
                acc = k == 0 ? cc * h[k] : __builtin_fmaf(cc, h[k], acc);
            }
            pv[i] = acc;
        });
        *reinterpret_cast<float4*>(sp + 4 * Q) = float4{pv[0], pv[1], pv[2], pv[3]};
    };

    // the same software pipeline as the 16-state kernel, per 16-step chunk
    const int64_t nch = (L + kLwT - 1) / kLwT;
    const bool ragged = L % kLwT != 0;
    {
        Raw w0;
        fetch(0, ragged && nch == 1, w0);
        uint32_t v[SPT][4];
        stage_load(0, ragged && nch == 1, v);
        stage_store(0, v);
        prologue(w0);
    }
    for (int64_t k = 0; k < nch; ++k) {
        const uint32_t t0 = (uint32_t)(k * kLwT);
        const int buf = (int)(k & 1);
        const int64_t kn = k + 1 < nch ? k + 1 : k;
        const bool next_tail = ragged && kn == nch - 1;
        __syncthreads();  // chunk k staged; every wave is done with chunk k-1's buffer
        uint32_t sv[SPT][4];
        stage_load(kn, next_tail, sv);
        Raw nx;
        fetch(kn, next_tail, nx);
        float hk[S];  // the states before step t0 (segment k), stored with y
#pragma unroll
        for (int s = 0; s < S; ++s) hk[s] = h[s];
        bl_for_ls<0, 4>([&](auto qc) __attribute__((always_inline)) { steps4(buf, qc); });
        stage_store(buf ^ 1, sv);
        const float u0 = uv, g0 = gz;
        prologue(nx);
        __builtin_amdgcn_wave_barrier();
        // step j: the row's 16 lanes in order
        float y = chan[j];
#pragma unroll
        for (int m = 1; m < 16; ++m) y += chan[m * kLwRowP + j];
        __builtin_amdgcn_wave_barrier();
        const float o = __builtin_fmaf(Dv, u0, y) * g0;
        if (!(ragged && k == nch - 1)) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), yr, (int)oy_l, (int)(t0 * 4u), 0);
        } else {
            const uint32_t a = t0 + j < (uint32_t)L ? oy_l : kLsDropBase;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), yr, (int)a, (int)(t0 * 4u), 0);
        }
        if constexpr (CK) {
#pragma unroll
            for (int s = 0; s < S; ++s)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hk[s]), ckr, (int)(ock + 64u * s),
                                                      (int)(t0 * (N / 4)), 0);
        }
    }
    if (p.last_state && valid) {
#pragma unroll
        for (int s = 0; s < S; ++s) p.last_state[b * p.sls_b + d * p.sls_d + j + 16 * s] = h[s];
    }
}

// ---------------------------------------------------------------------------------------------
// host side

// The lane-per-state kernels take dstate 16, 32 or 64, and shapes whose byte offsets within a
// wave's rows (u, delta, z, y) and within a batch's B / C fit 31 bits.
inline bool ls_eligible(const ScanParams& q, int64_t es) {
    if (q.dstate != 16 && q.dstate != 32 && q.dstate != 64) return false;
    const int64_t lim = (int64_t)1 << 31;
    const auto rows_ok = [&](const void* ptr, int64_t sd, int64_t e) {
        return ptr == nullptr || (3 * sd + q.len) * e < lim;
    };
    if (!rows_ok(q.u, q.su_d, es) || !rows_ok(q.delta, q.sdt_d, es) || !rows_ok(q.z, q.sz_d, es)) return false;
    if (!rows_ok(q.y, q.sy_d, 4)) return false;
    if (((q.dstate - 1) * q.sB_n + q.len) * es >= lim || ((q.dstate - 1) * q.sC_n + q.len) * es >= lim) return false;
    if (q.batch * q.dim > 0x7fffffff) return false;
    if (q.ck && q.ck_nseg * 16 * q.dstate >= lim) return false;  // a wave's saved states: 4 rows x nseg x N floats
    return true;
}

template <typename T, bool SP, bool HZ, bool VEC, bool CK, bool ZOH>
int launch_ls_cfg(const ScanParams& q, hipStream_t stream) {
    const void* fn;
    int64_t per_group;
    switch (q.dstate) {
        case 16: fn = reinterpret_cast<const void*>(&scan_ls_kernel<T, SP, HZ, VEC, CK, ZOH>); per_group = 16; break;
        case 32: fn = reinterpret_cast<const void*>(&scan_ls_wide_kernel<T, 32, SP, HZ, VEC, CK, ZOH>); per_group = 16; break;
        default: fn = reinterpret_cast<const void*>(&scan_ls_wide_kernel<T, 64, SP, HZ, VEC, CK, ZOH>); per_group = 16; break;
    }
    void* args[] = {const_cast<ScanParams*>(&q)};
    const int64_t groups = q.batch * ((q.dim + per_group - 1) / per_group);
    return hipLaunchKernel(fn, dim3((unsigned)groups), dim3(64 * kLsWaves), args, 0, stream) == hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

template <typename T, bool SP, bool HZ, bool VEC>
int launch_ls_ck(const ScanParams& q, hipStream_t stream) {
    // saving the segment states is a separate instantiation: the plain forward issues no stores
    // for it; so is the zero-order hold
    if (q.zoh_b)
        return q.ck ? launch_ls_cfg<T, SP, HZ, VEC, true, true>(q, stream)
                    : launch_ls_cfg<T, SP, HZ, VEC, false, true>(q, stream);
    return q.ck ? launch_ls_cfg<T, SP, HZ, VEC, true, false>(q, stream)
                : launch_ls_cfg<T, SP, HZ, VEC, false, false>(q, stream);
}

template <typename T, bool SP, bool HZ>
int launch_ls_vec(const ScanParams& q, hipStream_t stream) {
    // B / C rows 4-element aligned: one vector load per 4 staged steps
    const auto al = [](const void* ptr, int64_t sb, int64_t sn) {
        return reinterpret_cast<uintptr_t>(ptr) % (4 * sizeof(T)) == 0 && sb % 4 == 0 && sn % 4 == 0;
    };
    if (al(q.B, q.sB_b, q.sB_n) && al(q.C, q.sC_b, q.sC_n)) return launch_ls_ck<T, SP, HZ, true>(q, stream);
    return launch_ls_ck<T, SP, HZ, false>(q, stream);
}

template <typename T>
int launch_ls(const ScanParams& q, hipStream_t stream) {
    if (!ls_eligible(q, sizeof(T))) return MAMBA_SCAN_ERR_UNSUPPORTED;
    const bool sp = q.softplus != 0, hz = q.z != nullptr;
    if (sp && hz) return launch_ls_vec<T, true, true>(q, stream);
    if (sp) return launch_ls_vec<T, true, false>(q, stream);
    if (hz) return launch_ls_vec<T, false, true>(q, stream);
    return launch_ls_vec<T, false, false>(q, stream);
}

}  // namespace mscan
