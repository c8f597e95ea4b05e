// Device-side helpers shared by the selective-scan kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

// Everything a kernel needs, passed by value. Strides are in elements.
struct ScanParams {
    const void* u;
    const void* delta;
    const void* z;
    const void* B;
    const void* C;
    const float* A;
    const float* D;
    const float* bias;
    const float* h0;
    float* y;
    float* last_state;
    int64_t batch, dim, len, dstate;
    int64_t su_b, su_d, sdt_b, sdt_d, sz_b, sz_d;
    int64_t sB_b, sB_n, sC_b, sC_n;
    int64_t sy_b, sy_d;
    int64_t sh0_b, sh0_d, sls_b, sls_d;
    int64_t sA_d, sD, sbias;
    int softplus;
    int zoh_b;  // B discretised by zero-order hold instead of dt * B
    float* ck;        // or NULL: the state before every 16-step segment, (batch, dim, ck_nseg, dstate)
    int64_t ck_nseg;  // ceil(len / 16)
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage types: fp32, or bf16 held as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v.bits << 16); }

// Hardware transcendentals: v_exp_f32 is 2^x, v_log_f32 is log2(x), v_rcp_f32 is 1/x.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = ln(1 + e^x) = max(x, 0) + log1p(e) with e = e^-|x| in (0, 1].
// log1p(e): w = 1 + e is rounded, and r = e - (w - 1) is that rounding error exactly (w - 1 is
// exact for w in [1, 2]). Then log1p(e) = ln(w) + ln(1 + r/w) = ln(w) + r to within |r|*e + r^2,
// i.e. below 2^-24 relative: no division and no special case for w == 1 (then r = e).
__device__ __forceinline__ float softplus_f(float x) {
    const float e = hw_exp2(-__builtin_fabsf(x) * kLog2e);
    const float w = 1.0f + e;
    const float r = e - (w - 1.0f);
    return __builtin_fmaf(hw_log2(w), kLn2, r + __builtin_fmaxf(x, 0.0f));
}

// dt from the biased delta: softplus, or exp when the softplus flag is clear.
__device__ __forceinline__ float delta_to_dt(float x, int softplus) {
    return softplus ? softplus_f(x) : hw_exp2(x * kLog2e);
}

// Zero-order-hold coefficient of B for one diagonal state, (e^{dt A} - 1) / A, given x = dt * A,
// dA = e^x (already computed for the decay) and invA = 1 / A (0 where A = 0). For |x| < 1/16 the
// series dt (1 + x/2 + x^2/6 + x^3/24 + x^4/120), whose truncation is below 2^-29 relative and
// which is exact at A = 0 (dt); above, (dA - 1) * invA, where |dA - 1| > 0.06 keeps the
// cancellation under 2^-20 relative. The discretisation of "手把手用PyTorch实现Mamba的SSM层…" §2.1,
// B_d = A^-1 (e^{A dt} - I) B, for a diagonal A.
__device__ __forceinline__ float zoh_coef_f(float dt, float x, float dA, float invA) {
    const float p = __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 120.0f, 1.0f / 24.0f), 1.0f / 6.0f), 0.5f), 1.0f);
    const float small = dt * p;
    const float big = (dA - 1.0f) * invA;
    return __builtin_fabsf(x) < 0.0625f ? small : big;
}

// The same coefficient from the decay's exponent in base 2, x2 = dt * A * log2(e), as the
// lane-per-state kernels have it, and ia = 1 / A (0 where A = 0): for |dt A| < 1/16 the series
// dt (1 + x/2 + x^2/6 + x^3/24) with its coefficients scaled to x2 (truncation below 2^-22
// relative; exact, dt, at A = 0), above it dA ia - ia in one rounding (cancellation under 2^-20
// relative, as above). Three FMAs, a multiply, an FMA and a select beside the Euler term.
constexpr float kZohS1 = 0.34657359027997264f;   // ln 2 / 2
constexpr float kZohS2 = 0.080075502319700240f;  // (ln 2)^2 / 6
constexpr float kZohS3 = 0.013876027166205392f;  // (ln 2)^3 / 24
constexpr float kZohX2 = 0.090168440055560210f;  // 1/16 in base-2 exponent units: 1 / (16 ln 2)
__device__ __forceinline__ float zoh_coef2_f(float dt, float x2, float dA, float ia) {
    const float p = __builtin_fmaf(x2, __builtin_fmaf(x2, __builtin_fmaf(x2, kZohS3, kZohS2), kZohS1), 1.0f);
    const float small = dt * p;
    const float big = __builtin_fmaf(dA, ia, -ia);
    return __builtin_fabsf(x2) < kZohX2 ? small : big;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu_f(float z) { return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e)); }

}  // namespace mscan
