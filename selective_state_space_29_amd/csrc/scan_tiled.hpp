// LDS-tiled, software-pipelined selective-scan kernel for gfx950.
//
// Work decomposition. A workgroup owns 64 consecutive channels d of one batch b (one channel per
// lane) and walks the sequence in chunks of TC steps. Its W waves split the N states: wave w
// carries states n = w*S .. w*S+S-1 for all 64 channels, in registers, across the whole sequence.
//   * B[b, n, t] and C[b, n, t] are then the same for every lane of a wave: they are read with
//     scalar loads into SGPRs and enter the VALU as scalar operands at no per-lane cost.
//   * The per-(channel, step) work that does not depend on n - the biased softplus/exp of delta,
//     dt*u, the skip D*u and the silu gate - is done once per chunk by the whole workgroup
//     (each thread takes QS consecutive steps of one channel, so global accesses are vectors
//     along L) and shared through LDS.
// Per element (b, d, t, n) the inner loop is then the minimum the recurrence needs:
//   v_mul (dt * A*log2e), v_exp (2^x), v_mul (dt*u * B), v_fma (h = dA*h + dBu), v_fma (y += C*h)
// with fp32 state kept in VGPRs. The W partial outputs of a step are summed in LDS in wave order
// (deterministic), then skip and gate are applied and y is stored as vectors.
// This is the recurrence of "Mamba代码实战…" §3.1-§3.3 with the output contraction of
// "Mamba-minimal项目解析…" 关键技术点 1, fused so that no (B, D, L, N) tensor is ever formed (the
// page itself materialises dA and dB, §3.1).
//
// Pipeline. LDS holds two buffers of dt/dt*u and two of partial outputs. Between two barriers
// every wave runs, as one straight-line block the compiler can interleave:
//   main(c)       dt, dt*u of chunk c from LDS -> recurrence -> partial outputs of chunk c
//   epilogue(c-1) partial outputs of chunk c-1 -> sum, skip, gate -> y
//   prologue(c+1) raw inputs of chunk c+1 (loaded one interval earlier) -> dt, dt*u into LDS
// so one barrier per chunk separates producers from consumers. Inside main(c) the LDS reads
// come first; the chunk's B/C scalar loads are issued only after they complete (scalar loads and
// LDS share one wait counter) and their latency is covered by the chunk's exps, which do not
// need B/C.
#pragma once

#include <type_traits>

#include "../../include/mamba_scan.h"
#include "common.hpp"

namespace mscan {

typedef const __attribute__((address_space(4))) uint32_t* cptr32;  // scalar-load pointer
typedef const __attribute__((address_space(4))) float* cptrf;

// QS consecutive steps of one tensor row, as loaded from global memory.
template <typename T, int QS>
struct Vec;

template <int QS>
struct Vec<float, QS> {
    float v[QS];
    __device__ __forceinline__ void load(const float* p) {
        if constexpr (QS == 4) {
            const float4 x = *reinterpret_cast<const float4*>(p);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else if constexpr (QS == 2) {
            const float2 x = *reinterpret_cast<const float2*>(p);
            v[0] = x.x; v[1] = x.y;
        } else {
            v[0] = p[0];
        }
    }
    __device__ __forceinline__ void load_tail(const float* p, int n) {
#pragma unroll
        for (int j = 0; j < QS; ++j) v[j] = j < n ? p[j] : 0.0f;
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int j = 0; j < QS; ++j) v[j] = 0.0f;
    }
    __device__ __forceinline__ float get(int j) const { return v[j]; }
};

template <int QS>
struct Vec<bf16_t, QS> {
    static constexpr int NW = (QS + 1) / 2;  // 32-bit words
    uint32_t w[NW];
    __device__ __forceinline__ void load(const bf16_t* p) {
        if constexpr (QS == 4) {
            const uint2 x = *reinterpret_cast<const uint2*>(p);
            w[0] = x.x; w[1] = x.y;
        } else if constexpr (QS == 2) {
            w[0] = *reinterpret_cast<const uint32_t*>(p);
        } else {
            w[0] = p[0].bits;
        }
    }
    __device__ __forceinline__ void load_tail(const bf16_t* p, int n) {
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const uint32_t lo = (2 * k) < n ? p[2 * k].bits : 0u;
            const uint32_t hi = (2 * k + 1) < n && (2 * k + 1) < QS ? p[2 * k + 1].bits : 0u;
            w[k] = lo | (hi << 16);
        }
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int k = 0; k < NW; ++k) w[k] = 0u;
    }
    __device__ __forceinline__ float get(int j) const {
        const uint32_t x = w[j >> 1];
        return __uint_as_float((j & 1) ? (x & 0xffff0000u) : (x << 16));
    }
};

// QS floats to/from LDS
template <int QS>
__device__ __forceinline__ void lds_store(float* p, const float (&v)[QS]) {
    if constexpr (QS == 4) *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else if constexpr (QS == 2) *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    else p[0] = v[0];
}
template <int QS>
__device__ __forceinline__ void lds_load(const float* p, float (&v)[QS]) {
    if constexpr (QS == 4) {
        const float4 x = *reinterpret_cast<const float4*>(p);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else if constexpr (QS == 2) {
        const float2 x = *reinterpret_cast<const float2*>(p);
        v[0] = x.x; v[1] = x.y;
    } else {
        v[0] = p[0];
    }
}

// TC wave-uniform values of one B (or C) row starting at element `off`, through the scalar cache,
// kept in their storage format until used (packed bf16 pairs stay packed: half the SGPRs).
// For bf16 `off` is even (checked on the host), so the values are TC/2 aligned dwords.
template <typename T, int TC>
struct URow;

template <int TC>
struct URow<float, TC> {
    float v[TC];
    __device__ __forceinline__ void load(const float* base, int64_t off) {
        const cptrf p = (cptrf)(base + off);
#pragma unroll
        for (int t = 0; t < TC; ++t) v[t] = p[t];
    }
    __device__ __forceinline__ float get(int t) const { return v[t]; }
};

template <int TC>
struct URow<bf16_t, TC> {
    uint32_t w[TC / 2];
    __device__ __forceinline__ void load(const bf16_t* base, int64_t off) {
        const cptr32 p = (cptr32)(base + off);
#pragma unroll
        for (int k = 0; k < TC / 2; ++k) w[k] = p[k];
    }
    __device__ __forceinline__ float get(int t) const {
        const uint32_t x = w[t >> 1];
        return __uint_as_float((t & 1) ? (x & 0xffff0000u) : (x << 16));
    }
};
// One value, per lane (same address in every lane); used in the tail chunk only.
__device__ __forceinline__ float lane_load(const float* base, int64_t off) { return base[off]; }
__device__ __forceinline__ float lane_load(const bf16_t* base, int64_t off) { return to_f32(base[off]); }

template <bool SOFTPLUS>
__device__ __forceinline__ float dt_of(float x) {
    if constexpr (SOFTPLUS) return softplus_f(x);
    else return hw_exp2(x * kLog2e);
}

#ifndef MSCAN_TOUCH_BC
#define MSCAN_TOUCH_BC 0
#endif
constexpr bool kTouchBC = MSCAN_TOUCH_BC;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Buffer-resource word 3 for untyped 32-bit buffer accesses on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;
// An offset no buffer resource here reaches: stores to it are dropped by the hardware.
constexpr uint32_t kDropOffset = 0xFFFFFFF0u;

template <int QS>
__device__ __forceinline__ void buffer_store(const float (&v)[QS], __amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (QS == 4)
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])}, r,
            (int)off, 0, 0);
    else if constexpr (QS == 2)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v[0]), __float_as_uint(v[1])}, r, (int)off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, (int)off, 0, 0);
}

template <typename T, int S, int W, int TC, bool SOFTPLUS, bool HAS_Z, bool EXACT, bool ZOH>
__global__ __launch_bounds__(64 * W) void scan_tiled_kernel(ScanParams p) {
    constexpr int QS = TC / W;    // steps per thread in prologue/epilogue
    constexpr int NQ = TC / QS;   // step groups per channel and chunk (= W)
    constexpr int ROWP = TC + 4;  // padded LDS row (floats) of one channel
    static_assert(TC % W == 0 && (QS == 1 || QS == 2 || QS == 4) && TC % 4 == 0, "bad tiling");

    __shared__ float s_dt[64 * ROWP];
    __shared__ float s_dtu[64 * ROWP];
    __shared__ float s_yp[W * 64 * ROWP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t ngroups = (p.dim + 63) / 64;
    const int64_t b = blockIdx.x / ngroups;
    const int64_t d0 = (blockIdx.x - b * ngroups) * 64;
    const int64_t L = p.len;
    const int nbase = wave * S;
    const bool wave_live = EXACT || nbase < (int)p.dstate;  // the host guarantees N % S == 0

    // ---- prologue/epilogue role: QS consecutive steps of one channel ----
    const int pr = tid / NQ;
    const int pq = tid - pr * NQ;
    const int64_t pd = d0 + pr;
    const bool pvalid = pd < p.dim;
    const int64_t pdc = pvalid ? pd : 0;  // rows past dim read row 0 and store nothing
    const float pbias = p.bias ? p.bias[pdc * p.sbias] : 0.0f;
    const float pskip = p.D ? p.D[pdc * p.sD] : 0.0f;
    const T* pu = static_cast<const T*>(p.u) + b * p.su_b + pdc * p.su_d + QS * pq;
    const T* pdl = static_cast<const T*>(p.delta) + b * p.sdt_b + pdc * p.sdt_d + QS * pq;
    const T* pz = HAS_Z ? static_cast<const T*>(p.z) + b * p.sz_b + pdc * p.sz_d + QS * pq : nullptr;
    const int prow = pr * ROWP + QS * pq;
    // y: one buffer resource over this workgroup's rows, moved along L chunk by chunk
    const int64_t rows_here = (p.dim - d0) < 64 ? (p.dim - d0) : 64;
    float* ybase = p.y + b * p.sy_b + d0 * p.sy_d;
    const int64_t ybytes = ((rows_here - 1) * p.sy_d + L) * 4;  // < 2^31, checked on the host
    const uint32_t yoff = pvalid ? (uint32_t)((pr * p.sy_d + QS * pq) * 4) : kDropOffset;

    // ---- main-loop role: this lane's channel, this wave's states ----
    const int64_t dm = d0 + lane;
    const bool mvalid = dm < p.dim;
    float a2[S], h[S], an[S], ian[S];  // an, ian: A and 1/A (zero-order-hold B only)
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = nbase + s;
        a2[s] = an[s] = ian[s] = 0.0f;
        h[s] = 0.0f;
        if (wave_live && mvalid) {
            an[s] = p.A[dm * p.sA_d + n];
            a2[s] = an[s] * kLog2e;
            if constexpr (ZOH) ian[s] = an[s] != 0.0f ? 1.0f / an[s] : 0.0f;
            if (p.h0) h[s] = p.h0[b * p.sh0_b + dm * p.sh0_d + n];
        }
    }
    const int nclamp = wave_live ? nbase : 0;  // idle waves point at valid rows, load nothing
    const T* Bw = static_cast<const T*>(p.B) + b * p.sB_b + (int64_t)nclamp * p.sB_n;
    const T* Cw = static_cast<const T*>(p.C) + b * p.sC_b + (int64_t)nclamp * p.sC_n;
    const int64_t sBn = p.sB_n, sCn = p.sC_n;
    float* yrow = &s_yp[(wave * 64 + lane) * ROWP];
    const float* dtrow = &s_dt[lane * ROWP];
    const float* dturow = &s_dtu[lane * ROWP];

    const int64_t nchunks = (L + TC - 1) / TC;

    // Raw inputs are fetched two chunks ahead of their prologue, into one of two register sets
    // (chunk c uses set c & 1); the steady loop below is unrolled by two so the set index is a
    // compile-time constant.
    Vec<T, QS> ru[2], rdl[2], rz[2];
    auto fetch = [&](int64_t c, auto set_tag) __attribute__((always_inline)) {
        constexpr int k = decltype(set_tag)::value;
        const int64_t t0 = c * TC;
        const int64_t nleft64 = L - t0 - QS * pq;
        if (nleft64 >= QS) {
            ru[k].load(pu + t0);
            rdl[k].load(pdl + t0);
            if constexpr (HAS_Z) rz[k].load(pz + t0);
        } else {
            const int nleft = (int)(nleft64 > 0 ? nleft64 : 0);
            ru[k].load_tail(pu + t0, nleft);
            rdl[k].load_tail(pdl + t0, nleft);
            if constexpr (HAS_Z) rz[k].load_tail(pz + t0, nleft);
        }
    };

    // prologue of chunk c: dt and dt*u (u alone with zero-order-hold B) into LDS; keeps u and z
    // for its epilogue
    auto prologue = [&](int64_t c, auto set_tag, float (&cu)[QS], float (&cz)[QS]) {
        constexpr int k = decltype(set_tag)::value;
        const int64_t left = L - c * TC - QS * pq;
        const int nvalid = (int)(left < QS ? (left > 0 ? left : 0) : QS);
        float dt[QS], dtu[QS];
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            cu[j] = ru[k].get(j);
            cz[j] = HAS_Z ? rz[k].get(j) : 0.0f;
            const float v = dt_of<SOFTPLUS>(rdl[k].get(j) + pbias);
            dt[j] = (j < nvalid) ? v : 0.0f;  // steps beyond L leave h unchanged
            dtu[j] = ZOH ? cu[j] : dt[j] * cu[j];
        }
        lds_store<QS>(&s_dt[prow], dt);
        lds_store<QS>(&s_dtu[prow], dtu);
    };

    // epilogue of chunk c: the W partial outputs are read before the mid-chunk barrier; the sum,
    // skip and gate follow, then the store
    auto epi_read = [&](float (&acc)[QS]) {
        lds_load<QS>(&s_yp[prow], acc);
#pragma unroll
        for (int w = 1; w < W; ++w) {
            float v[QS];
            lds_load<QS>(&s_yp[w * 64 * ROWP + prow], v);
#pragma unroll
            for (int j = 0; j < QS; ++j) acc[j] += v[j];
        }
    };
    auto epi_math = [&](float (&acc)[QS], const float (&cu)[QS], const float (&cz)[QS]) {
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            acc[j] = __builtin_fmaf(pskip, cu[j], acc[j]);
            if constexpr (HAS_Z) acc[j] *= silu_f(cz[j]);
        }
    };
    auto y_rsrc = [&](int64_t c) __attribute__((always_inline)) {
        const int64_t t0 = c * TC;
        return __builtin_amdgcn_make_buffer_rsrc(ybase + t0, 0, (int)(ybytes - t0 * 4), kBufferWord3);
    };
    auto epi_store_full = [&](int64_t c, const float (&acc)[QS]) { buffer_store<QS>(acc, y_rsrc(c), yoff); };
    auto epi_store_tail = [&](int64_t c, const float (&acc)[QS]) {
        const int64_t left = L - c * TC - QS * pq;
        if (!pvalid || left <= 0) return;
        float* yp = ybase + pr * p.sy_d + QS * pq + c * TC;
#pragma unroll
        for (int j = 0; j < QS; ++j)
            if (j < left) yp[j] = acc[j];
    };

    // main(c), full chunk. dt and dt*u are read into registers before the mid-chunk barrier;
    // after it no LDS read is left in the chunk, so the B/C scalar loads go out first and the
    // decays (which need no B/C) plus the epilogue/prologue work cover their latency.
    float dtv[TC], dtuv[TC];
    auto main_read = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < TC / 4; ++q) {
            const float4 x = *reinterpret_cast<const float4*>(dtrow + 4 * q);
            const float4 y = *reinterpret_cast<const float4*>(dturow + 4 * q);
            dtv[4 * q] = x.x; dtv[4 * q + 1] = x.y; dtv[4 * q + 2] = x.z; dtv[4 * q + 3] = x.w;
            dtuv[4 * q] = y.x; dtuv[4 * q + 1] = y.y; dtuv[4 * q + 2] = y.z; dtuv[4 * q + 3] = y.w;
        }
    };
    URow<T, TC> bv[S], cv[S];
    float dA[S][TC];
    auto main_issue = [&](int64_t c) __attribute__((always_inline)) {
        const int64_t t0 = c * TC;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            bv[s].load(Bw, s * sBn + t0);
            cv[s].load(Cw, s * sCn + t0);
        }
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int t = 0; t < TC; ++t) dA[s][t] = hw_exp2(dtv[t] * a2[s]);
    };
    // Touch the first and last dword of chunk c's B/C rows with scalar loads, so that they are in
    // the scalar cache when main(c) loads them. Called once chunk c-1's B/C have arrived, its
    // loads complete during the rest of the chunk; the values only feed an empty asm sink.
    auto bc_touch = [&](int64_t c) __attribute__((always_inline)) {
        const int64_t t0 = c * TC;
        uint32_t sink = 0;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const cptr32 pb = (cptr32)(Bw + s * sBn + t0);
            const cptr32 pc = (cptr32)(Cw + s * sCn + t0);
            constexpr int last = (TC * (int)sizeof(T)) / 4 - 1;
            sink ^= pb[0] ^ pb[last] ^ pc[0] ^ pc[last];
        }
        return sink;
    };
    auto main_recur = [&](int64_t c_next) __attribute__((always_inline)) {
        uint32_t sink = 0;
#pragma unroll
        for (int q = 0; q < TC / 4; ++q) {
            float yq[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 4 * q + j;
                float yv = 0.0f;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    float inc;
                    if constexpr (ZOH)
                        inc = zoh_coef_f(dtv[t], dtv[t] * an[s], dA[s][t], ian[s]) * dtuv[t] * bv[s].get(t);
                    else
                        inc = dtuv[t] * bv[s].get(t);
                    h[s] = __builtin_fmaf(dA[s][t], h[s], inc);
                    yv = __builtin_fmaf(cv[s].get(t), h[s], yv);
                }
                yq[j] = yv;
            }
            *reinterpret_cast<float4*>(yrow + 4 * q) = make_float4(yq[0], yq[1], yq[2], yq[3]);
            if (kTouchBC && q == 0 && c_next >= 0) {
                __builtin_amdgcn_sched_barrier(0);
                sink = bc_touch(c_next);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __asm__ volatile("" ::"s"(sink));
    };
    // main(c) for the last, partial chunk: one step at a time, B/C through per-lane loads
    auto main_tail = [&](int64_t c, int steps) __attribute__((always_inline)) {
        const int64_t t0 = c * TC;
        for (int i = 0; i < steps; ++i) {
            const float dt = dtrow[i], dtu = dturow[i];
            float yv = 0.0f;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const float bvv = lane_load(Bw, s * sBn + t0 + i);
                const float cvv = lane_load(Cw, s * sCn + t0 + i);
                const float d = hw_exp2(dt * a2[s]);
                const float inc = ZOH ? zoh_coef_f(dt, dt * an[s], d, ian[s]) * dtu * bvv : dtu * bvv;
                h[s] = __builtin_fmaf(d, h[s], inc);
                yv = __builtin_fmaf(cvv, h[s], yv);
            }
            yrow[i] = yv;
        }
    };
    auto zero_partials = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < TC / 4; ++q)
            *reinterpret_cast<float4*>(yrow + 4 * q) = make_float4(0.f, 0.f, 0.f, 0.f);
    };

    // u and z of the chunk whose epilogue runs next (cur) and of the one after it (nxt)
    float cu_cur[QS], cz_cur[QS], cu_nxt[QS], cz_nxt[QS];
#pragma unroll
    for (int j = 0; j < QS; ++j) cu_nxt[j] = cz_nxt[j] = 0.0f;
    auto rotate = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            cu_cur[j] = cu_nxt[j];
            cz_cur[j] = cz_nxt[j];
        }
    };
    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, 1>;

    fetch(0, Set0());
    if (nchunks > 1) fetch(1, Set1());
    prologue(0, Set0(), cu_cur, cz_cur);
    if (nchunks > 2) fetch(2, Set0());

    // chunk 0: no epilogue yet
    {
        const bool full = TC <= L;
        __syncthreads();
        if (full) main_read();
        __syncthreads();
        if (nchunks > 1) prologue(1, Set1(), cu_nxt, cz_nxt);
        if (nchunks > 3) fetch(3, Set1());
        if (!wave_live) zero_partials();
        else if (full) { main_issue(0); main_recur(nchunks > 1 ? 1 : -1); }
        else main_tail(0, (int)L);
    }

    // steady state: chunks 1 .. nchunks-2 are full; epilogue(c-1) and prologue(c+1) run in the
    // same straight-line block as main(c). Chunk c's prologue consumes raw set (c+1)&1, which is
    // refilled at once with chunk c+3.
    auto steady = [&](int64_t c, auto set_tag) __attribute__((always_inline)) {
        __syncthreads();  // prologue(c) and partial outputs of c-1 are in LDS
        float acc[QS];
        if (wave_live) main_read();
        epi_read(acc);
        __syncthreads();  // every wave holds its reads: LDS may be overwritten from here on
        if (wave_live) main_issue(c);
        epi_math(acc, cu_cur, cz_cur);
        rotate();
        prologue(c + 1, set_tag, cu_nxt, cz_nxt);
        if (c + 3 < nchunks) fetch(c + 3, set_tag);
        if (wave_live) main_recur(c + 1);
        else zero_partials();
        epi_store_full(c - 1, acc);
    };
    int64_t c = 1;
    for (; c + 2 < nchunks; c += 2) {
        steady(c, Set0());      // prologue(c+1), c+1 even
        steady(c + 1, Set1());  // prologue(c+2), c+2 odd
    }
    if (c + 1 < nchunks) {
        steady(c, Set0());
        ++c;
    }

    // last chunk (full or partial), with the epilogue of the one before it
    if (nchunks > 1) {
        const int64_t cl = nchunks - 1;
        const bool full = cl * TC + TC <= L;
        __syncthreads();
        float acc[QS];
        if (full && wave_live) main_read();
        epi_read(acc);
        __syncthreads();
        epi_math(acc, cu_cur, cz_cur);
        rotate();
        if (!wave_live) zero_partials();
        else if (full) { main_issue(cl); main_recur(-1); }
        else main_tail(cl, (int)(L - cl * TC));
        epi_store_full(cl - 1, acc);
    }
    __syncthreads();
    {
        float acc[QS];
        epi_read(acc);
        epi_math(acc, cu_cur, cz_cur);
        epi_store_tail(nchunks - 1, acc);
    }

    if (p.last_state && wave_live && mvalid) {
        float* ls = p.last_state + b * p.sls_b + dm * p.sls_d + nbase;
#pragma unroll
        for (int s = 0; s < S; ++s) ls[s] = h[s];
    }
}

// ---------------------------------------------------------------------------------------------
// host side

// States per wave for the 8-wave workgroup: N <= 8 -> 1 (waves n >= N idle), then 2, 4, 8.
inline int tiled_states_per_wave(int64_t N) {
    if (N <= 8) return 1;
    if (N <= 16) return 2;
    if (N <= 32) return 4;
    if (N <= 64) return 8;
    return 0;
}

inline bool aligned(const void* ptr, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(ptr) % bytes) == 0; }

template <typename T>
bool tiled_eligible(const ScanParams& q, int qs) {
    const int S = tiled_states_per_wave(q.dstate);
    if (S == 0 || q.dstate % S != 0) return false;
    const uintptr_t vec = sizeof(T) * qs;  // one thread's steps
    const auto rows_ok = [&](const void* ptr, int64_t sb, int64_t sd) __attribute__((always_inline)) {
        return ptr == nullptr || (aligned(ptr, vec) && sb % qs == 0 && sd % qs == 0);
    };
    if (!rows_ok(q.u, q.su_b, q.su_d) || !rows_ok(q.delta, q.sdt_b, q.sdt_d) || !rows_ok(q.z, q.sz_b, q.sz_d))
        return false;
    if (!aligned(q.y, 4 * qs) || q.sy_b % qs != 0 || q.sy_d % qs != 0) return false;
    // B/C are read as aligned dwords through the scalar cache
    if (!aligned(q.B, 4) || !aligned(q.C, 4)) return false;
    if (sizeof(T) == 2 && (q.sB_b % 2 || q.sB_n % 2 || q.sC_b % 2 || q.sC_n % 2)) return false;
    if (q.batch * ((q.dim + 63) / 64) > 0x7fffffff) return false;
    // y of one workgroup (64 rows) is addressed through a 32-bit buffer offset
    if ((63 * q.sy_d + q.len) * 4 >= ((int64_t)1 << 31)) return false;
    return true;
}

// Whether launch_tiled can run this case (its states-per-wave split and alignment rules).
template <typename T>
bool tiled_can_run(const ScanParams& q) {
    switch (tiled_states_per_wave(q.dstate)) {
        case 1: case 2: return tiled_eligible<T>(q, 4);
        case 4: return tiled_eligible<T>(q, 2);
        case 8: return tiled_eligible<T>(q, 1);
        default: return false;
    }
}

template <typename T, int S, int W, int TC, bool SP, bool HZ>
int launch_tiled_cfg(const ScanParams& q, hipStream_t stream) {
    const int64_t groups = q.batch * ((q.dim + 63) / 64);
    void* args[] = {const_cast<ScanParams*>(&q)};
    const bool exact = q.dstate == (int64_t)S * W;
    const void* fn =
        q.zoh_b ? (exact ? reinterpret_cast<const void*>(&scan_tiled_kernel<T, S, W, TC, SP, HZ, true, true>)
                         : reinterpret_cast<const void*>(&scan_tiled_kernel<T, S, W, TC, SP, HZ, false, true>))
                : (exact ? reinterpret_cast<const void*>(&scan_tiled_kernel<T, S, W, TC, SP, HZ, true, false>)
                         : reinterpret_cast<const void*>(&scan_tiled_kernel<T, S, W, TC, SP, HZ, false, false>));
    return hipLaunchKernel(fn, dim3((unsigned)groups), dim3(64 * W), args, 0, stream) == hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

template <typename T, int S, int W, int TC>
int launch_tiled_s(const ScanParams& q, hipStream_t stream) {
    if (!tiled_eligible<T>(q, TC / W)) return MAMBA_SCAN_ERR_UNSUPPORTED;
    const bool sp = q.softplus != 0, hz = q.z != nullptr;
    if (sp && hz) return launch_tiled_cfg<T, S, W, TC, true, true>(q, stream);
    if (sp) return launch_tiled_cfg<T, S, W, TC, true, false>(q, stream);
    if (hz) return launch_tiled_cfg<T, S, W, TC, false, true>(q, stream);
    return launch_tiled_cfg<T, S, W, TC, false, false>(q, stream);
}

// Chunk length per states-per-wave: S*TC values of B and of C sit in SGPRs at once
// (S*TC = 64: 32 SGPRs each as packed bf16 pairs).
template <typename T>
int launch_tiled(const ScanParams& q, const mamba_scan_ptrs*, uint32_t, hipStream_t stream) {
    switch (tiled_states_per_wave(q.dstate)) {
        case 1: return launch_tiled_s<T, 1, 8, 32>(q, stream);
        case 2: return launch_tiled_s<T, 2, 8, 32>(q, stream);
        case 4: return launch_tiled_s<T, 4, 8, 16>(q, stream);
        case 8: return launch_tiled_s<T, 8, 8, 8>(q, stream);
        default: return MAMBA_SCAN_ERR_UNSUPPORTED;
    }
}

}  // namespace mscan
