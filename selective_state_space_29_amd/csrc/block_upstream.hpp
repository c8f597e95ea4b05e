// The stages of a Mamba block in front of the selective scan, on gfx950, in one kernel:
//   u     = bf16(silu(causal depthwise conv1d(x)))                 (batch, dim, L)
//   x_dbl = bf16(x_proj u)      rows: dt_rank dt rows, then B, then C      (batch, J, L)
//   delta = bf16(dt_proj x_dbl[:dt_rank])                           (batch, dim, L)
// The layers are those of the MambaBlock listing of "告别'炼丹'：从Mamba-minimal入手…" §1.1
// (Conv1d with padding d_conv - 1, Linear(d_inner, dt_rank + 2 d_state), Linear(dt_rank, d_inner)),
// with the split order of "Mamba-minimal项目解析…" §5. The convolution is depthwise and causal and is
// followed by SiLU; dt_proj's bias is the scan's delta_bias and is not added here.
//
// One workgroup owns one batch and 64 consecutive steps, and loops over the channels in chunks
// of 256: each chunk's x rows are read once from HBM, convolved, written out as u and staged in
// LDS as [step][channel] bf16, where they are the left operand of the x projection on the matrix
// cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation; two waves per 16 output rows). After the
// last chunk the x projection is rounded to bf16, written out, and its dt rows (staged in LDS)
// feed the dt projection, again on the matrix cores, whose result is rounded and written as delta.
// The projections are small next to the bytes moved: the kernel is bound by HBM.
#pragma once

#include "common.hpp"

namespace mscan {

struct UpParams {
    const uint16_t* x;
    const float* conv_w;
    const float* conv_b;
    const uint16_t* w_x;
    const uint16_t* w_dt;
    uint16_t* u;
    uint16_t* xdbl;
    uint16_t* delta;
    int64_t batch, dim, len;
    int dstate, dt_rank;
};

constexpr int kUpTT = 64;          // steps per workgroup
constexpr int kUpKD = 256;         // channels per chunk
constexpr int kUpThreads = 1024;   // 16 waves: 4 per SIMD
constexpr int kUpUS = kUpKD + 8;   // LDS row of the u tile, in bf16: [step][channel]
constexpr int kUpDS = 64 + 8;      // LDS row of the dt tile, in bf16: [step][dt row]
constexpr int kUpPrefetch = 1;     // chunks of loads in flight ahead of the one being convolved
constexpr int kUpGroup = 2;        // channel tiles of the dt projection per group of w_dt loads
constexpr int kUpMaxDim = 4096;    // channels whose conv weights fit the LDS staging area

typedef __bf16 up_bf16x8 __attribute__((ext_vector_type(8)));
typedef float up_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float up_widen(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

typedef __bf16 up_bf16x2 __attribute__((ext_vector_type(2)));
// Two fp32 values rounded to bf16 (nearest, ties to even: v_cvt_pk_bf16_f32), packed lo | hi << 16.
__device__ __forceinline__ uint32_t up_pack_bf16(float lo, float hi) {
    const up_bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ up_bf16x8 up_frag(uint4 v) { return __builtin_bit_cast(up_bf16x8, v); }

__device__ __forceinline__ up_f32x4 up_mfma(up_bf16x8 a, up_bf16x8 b, up_f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Buffer resources over one tensor (raw, untyped 32-bit accesses). Every global access of the
// kernel goes through one: an offset at or past the end reads 0 and drops a write, so masked
// lanes use kUpDrop instead of a branch. Branch-free accesses keep the count of outstanding
// vector-memory operations the same on every path, which lets the compiler wait for exactly the
// chunk it needs rather than for everything in flight.
constexpr int kUpWord3 = 0x00020000;
constexpr uint32_t kUpDrop = 0xFFFFFFF0u;

typedef unsigned int up_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int up_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t up_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kUpWord3);
}
__device__ __forceinline__ uint2 up_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const up_u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 up_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const up_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float up_load4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void up_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lo, uint32_t hi) {
    __builtin_amdgcn_raw_buffer_store_b64(up_u32x2{lo, hi}, r, (int)off, 0, 0);
}

// K = d_conv (1..4); KS = dt-projection k-steps of 32 (dt_rank <= 32 * KS).
template <int K, int KS>
__global__ __launch_bounds__(kUpThreads) void upstream_kernel(UpParams p) {
    __shared__ __align__(16) uint16_t s_u[2][kUpTT * kUpUS];
    __shared__ __align__(16) uint16_t s_dt[kUpTT * kUpDS];
    __shared__ __align__(16) float s_cw[kUpMaxDim * 4];  // taps right-aligned: zeros before d_conv
    __shared__ float s_cb[kUpMaxDim];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t D = p.dim, L = p.len;
    const int R = p.dt_rank, J = p.dt_rank + 2 * p.dstate;
    const int64_t ntiles = (L + kUpTT - 1) / kUpTT;
    const int64_t b = blockIdx.x / ntiles;
    const int64_t t0 = (blockIdx.x - b * ntiles) * kUpTT;
    const int nchunks = (int)((D + kUpKD - 1) / kUpKD);

    // per-batch tensors are addressed with 32-bit byte offsets (checked on the host)
    const __amdgpu_buffer_rsrc_t rx = up_rsrc(p.x + b * D * L, D * L * 2);
    const __amdgpu_buffer_rsrc_t ru = up_rsrc(p.u + b * D * L, D * L * 2);
    const __amdgpu_buffer_rsrc_t rdl = up_rsrc(p.delta + b * D * L, D * L * 2);
    const __amdgpu_buffer_rsrc_t rxd = up_rsrc(p.xdbl + b * J * L, (int64_t)J * L * 2);
    const __amdgpu_buffer_rsrc_t rwx = up_rsrc(p.w_x, (int64_t)J * D * 2);
    const __amdgpu_buffer_rsrc_t rwdt = up_rsrc(p.w_dt, D * R * 2);
    const __amdgpu_buffer_rsrc_t rcw = up_rsrc(p.conv_w, D * K * 4);
    const __amdgpu_buffer_rsrc_t rcb = up_rsrc(p.conv_b ? p.conv_b : p.conv_w, p.conv_b ? D * 4 : 0);

    // dt rows past dt_rank enter the dt projection as zeros
    for (int i = tid; i < kUpTT * kUpDS / 8; i += kUpThreads)
        reinterpret_cast<uint4*>(s_dt)[i] = make_uint4(0u, 0u, 0u, 0u);
    // every channel's conv weights and bias, once per workgroup (dim <= kUpMaxDim), read with
    // contiguous loads four at a time: s_cw[4 d + k + 4 - K] = conv_w[d, k]; the 4 - K leading
    // taps of each channel are zero
    for (int64_t d = tid; d < D; d += kUpThreads)
#pragma unroll
        for (int k = 0; k < 4 - K; ++k) s_cw[d * 4 + k] = 0.0f;
    {
        const int64_t nw = D * K;
        for (int64_t i0 = 0; i0 < nw; i0 += 4 * kUpThreads) {
            float w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t i = i0 + tid + kUpThreads * r;
                w[r] = up_load4f(rcw, i < nw ? (uint32_t)(i * 4) : kUpDrop);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t i = i0 + tid + kUpThreads * r;
                if (i < nw) s_cw[(i / K) * 4 + (i % K) + 4 - K] = w[r];
            }
        }
        for (int64_t d0 = 0; d0 < D; d0 += 4 * kUpThreads) {
            float w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t d = d0 + tid + kUpThreads * r;
                w[r] = up_load4f(rcb, d < D ? (uint32_t)(d * 4) : kUpDrop);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t d = d0 + tid + kUpThreads * r;
                if (d < D) s_cb[d] = w[r];
            }
        }
    }

    // ---- convolution role: 4 channels x 4 steps per thread ----
    const int rg = tid >> 4;  // channels 4 rg .. 4 rg + 3 of the chunk
    const int tg = tid & 15;  // steps t0 + 4 tg .. + 3
    const int64_t tt = t0 + 4 * tg;
    const bool t_ok = tt < L;             // L % 4 == 0: all four steps exist or none
    const bool h_ok = t_ok && tt >= 4;    // the four steps before exist
    // byte offsets (32-bit: one batch of a tensor is below 2 GiB) of this thread's first
    // channel's steps in chunk 0; a channel is L * 2 bytes further, a chunk kUpKD * L * 2
    const uint32_t row_bytes = (uint32_t)(L * 2);
    const uint32_t off0 = (uint32_t)((4 * rg) * L * 2 + tt * 2);
    const uint32_t chunk_bytes = (uint32_t)kUpKD * row_bytes;

    struct Raw {
        uint2 own[4], halo[4];
    };
    // chunks past the last one are fetched too (every offset drops): the loop has no tail
    auto fetch = [&](int c, Raw& r) __attribute__((always_inline)) {
        const int nvalid = (int)(D - (int64_t)c * kUpKD);  // channels of chunk c that exist
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = t_ok && 4 * rg + i < nvalid;
            const uint32_t off = off0 + (uint32_t)c * chunk_bytes + (uint32_t)i * row_bytes;
            r.own[i] = up_load8(rx, ok ? off : kUpDrop);
            r.halo[i] = up_load8(rx, (ok && h_ok) ? off - 8u : kUpDrop);
        }
    };
    // u for the chunk: written to HBM and to the LDS tile (zeros for channels past dim)
    auto conv = [&](int c, const Raw& r, uint16_t* tile) __attribute__((always_inline)) {
        const int nvalid = (int)(D - (int64_t)c * kUpKD);
        uint32_t q[4][2];  // [channel][step pair] packed bf16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = t_ok && 4 * rg + i < nvalid;
            const int dc = ok ? c * kUpKD + 4 * rg + i : 0;
            const float4 w4 = *reinterpret_cast<const float4*>(&s_cw[dc * 4]);
            const float wk[4] = {w4.x, w4.y, w4.z, w4.w};
            const float bias = s_cb[dc];
            float xv[8];
            xv[0] = up_widen(r.halo[i].x & 0xFFFFu); xv[1] = up_widen(r.halo[i].x >> 16);
            xv[2] = up_widen(r.halo[i].y & 0xFFFFu); xv[3] = up_widen(r.halo[i].y >> 16);
            xv[4] = up_widen(r.own[i].x & 0xFFFFu);  xv[5] = up_widen(r.own[i].x >> 16);
            xv[6] = up_widen(r.own[i].y & 0xFFFFu);  xv[7] = up_widen(r.own[i].y >> 16);
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // output step tt + j sees x[tt + j - 3 .. tt + j]; taps past d_conv are zero
                float acc = bias;
#pragma unroll
                for (int k = 4 - K; k < 4; ++k) acc = __builtin_fmaf(wk[k], xv[1 + j + k], acc);
                v[j] = ok ? silu_f(acc) : 0.0f;
            }
            q[i][0] = up_pack_bf16(v[0], v[1]);
            q[i][1] = up_pack_bf16(v[2], v[3]);
            const uint32_t off = off0 + (uint32_t)c * chunk_bytes + (uint32_t)i * row_bytes;
            up_store8(ru, ok ? off : kUpDrop, q[i][0], q[i][1]);
        }
        // [step][channel] tile: step j of the four channels
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int sh = 16 * (j & 1);
            const uint32_t lo = ((q[0][j >> 1] >> sh) & 0xFFFFu) | ((q[1][j >> 1] >> sh) << 16);
            const uint32_t hi = ((q[2][j >> 1] >> sh) & 0xFFFFu) | ((q[3][j >> 1] >> sh) << 16);
            *reinterpret_cast<uint2*>(tile + (4 * tg + j) * kUpUS + 4 * rg) = make_uint2(lo, hi);
        }
    };

    // ---- x projection role: wave w owns x_dbl rows 16 (w % 8) .. + 15 and channel half w / 8 of
    // every chunk; the two halves' sums are added at the end. Waves whose rows do not exist load
    // nothing (every offset drops) and keep zero accumulators ----
    const int jt = wave & 7;
    const int kh = wave >> 3;
    const bool proj_wave = jt * 16 < J;
    const int jrow = jt * 16 + (lane & 15);
    const int kq = 8 * (lane >> 4);  // this lane's 8 consecutive k of a 32-wide k-step
    const bool jrow_ok = jrow < J;
    // dim % 8 == 0: a lane's 8 channels are all in or all out
    const uint32_t wx_off0 = jrow_ok ? (uint32_t)((jrow * D + kq) * 2) : 0x80000000u;  // past the end
    constexpr int KH = kUpKD / 2;  // channels per half chunk
    auto wx_fetch = [&](int c, uint4 (&f)[KH / 32]) __attribute__((always_inline)) {
        const int nvalid = (int)(D - (int64_t)c * kUpKD);
#pragma unroll
        for (int ks = 0; ks < KH / 32; ++ks) {
            const int k0 = KH * kh + 32 * ks;
            f[ks] = up_load16(rwx, k0 + kq < nvalid ? wx_off0 + (uint32_t)(c * kUpKD + k0) * 2u : kUpDrop);
        }
    };
    up_f32x4 acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = up_f32x4{0.f, 0.f, 0.f, 0.f};
    // x_dbl^T[t, j] += sum_d u^T[t, d] * w_x^T[d, j]: A = u tile rows (steps), B = w_x rows
    auto project = [&](const uint16_t* tile, const uint4 (&f)[KH / 32]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KH / 32; ++ks)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint4 a = *reinterpret_cast<const uint4*>(tile + (16 * m + (lane & 15)) * kUpUS + KH * kh + 32 * ks + kq);
                acc[m] = up_mfma(up_frag(a), up_frag(f[ks]), acc[m]);
            }
    };

    // PF chunks of loads in flight: a ring of PF + 1 register sets, the loop unrolled by PF + 1 so
    // that every set index is a compile-time constant. All loads of a chunk (x rows, w_x
    // fragments) are issued together, PF chunks ahead of their use: the vector-memory counter
    // drains in order, so a later-issued load of a nearer chunk would make the wait cover the far
    // ones too.
    constexpr int PF = kUpPrefetch;
    Raw raw[PF + 1];
    uint4 wxf[PF + 1][KH / 32];
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        fetch(k, raw[k]);
        wx_fetch(k, wxf[k]);
    }
    __syncthreads();  // conv weights and the zeroed dt tile are in LDS
    auto chunk = [&](int c, auto slot) __attribute__((always_inline)) {
        constexpr int P = decltype(slot)::value;  // = c % (PF + 1)
        constexpr int N = (P + PF) % (PF + 1);    // set of chunk c + PF
        fetch(c + PF, raw[N]);
        wx_fetch(c + PF, wxf[N]);
        conv(c, raw[P], s_u[c & 1]);
        __syncthreads();
        if (proj_wave) project(s_u[c & 1], wxf[P]);
    };
    for (int c = 0; c < nchunks; c += PF + 1) {
        chunk(c, std::integral_constant<int, 0>());
        chunk(c + 1, std::integral_constant<int, 1>());
        if constexpr (PF >= 2) chunk(c + 2, std::integral_constant<int, 2 % (PF + 1)>());
        if constexpr (PF >= 3) chunk(c + 3, std::integral_constant<int, 3 % (PF + 1)>());
    }

    // ---- the second half's sums onto the first (through LDS, over the u tile) ----
    __syncthreads();
    float* s_red = reinterpret_cast<float*>(s_u[0]);  // 8 x 64 lanes x 16 floats = 32 KB
    if (kh == 1 && proj_wave)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            *reinterpret_cast<float4*>(&s_red[((jt * 64 + lane) * 4 + m) * 4]) = make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
    __syncthreads();
    if (kh == 0 && proj_wave)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 o = *reinterpret_cast<const float4*>(&s_red[((jt * 64 + lane) * 4 + m) * 4]);
            acc[m][0] += o.x; acc[m][1] += o.y; acc[m][2] += o.z; acc[m][3] += o.w;
        }

    // ---- x_dbl out (first-half waves); its dt rows into LDS ----
    const int trow = 4 * (lane >> 4);  // this lane's 4 steps within each 16-step tile
    const bool xd_wave = kh == 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t lo = up_pack_bf16(acc[m][0], acc[m][1]), hi = up_pack_bf16(acc[m][2], acc[m][3]);
        const int64_t t = t0 + 16 * m + trow;
        up_store8(rxd, (xd_wave && jrow_ok && t < L) ? (uint32_t)((jrow * L + t) * 2) : kUpDrop, lo, hi);
        if (xd_wave && jrow < R) {
            s_dt[(16 * m + trow + 0) * kUpDS + jrow] = (uint16_t)(lo & 0xFFFFu);
            s_dt[(16 * m + trow + 1) * kUpDS + jrow] = (uint16_t)(lo >> 16);
            s_dt[(16 * m + trow + 2) * kUpDS + jrow] = (uint16_t)(hi & 0xFFFFu);
            s_dt[(16 * m + trow + 3) * kUpDS + jrow] = (uint16_t)(hi >> 16);
        }
    }
    __syncthreads();

    // ---- dt projection: delta^T[t, d] = sum_r dt^T[t, r] * w_dt^T[r, d]; wave w owns channel
    // tiles w, w + 16, ...; the dt^T fragments are the same for every tile ----
    constexpr int kW = kUpThreads / 64;
    uint4 dtf[4][KS];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            dtf[m][ks] = *reinterpret_cast<const uint4*>(s_dt + (16 * m + (lane & 15)) * kUpDS + 32 * ks + kq);
    const int64_t dtiles = (D + 15) / 16;
    // w_dt fragments of a group of kUpGroup channel tiles are loaded one group ahead of the
    // group whose delta is being stored; tiles past the last one load and store nothing
    auto wdt_fetch = [&](int64_t g, uint4 (&wf)[kUpGroup][KS]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kUpGroup; ++i) {
            const int64_t d = (wave + kW * (g * kUpGroup + i)) * 16 + (lane & 15);
            const uint32_t off = d < D ? (uint32_t)((d * R + kq) * 2) : 0x80000000u;  // past the end
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) wf[i][ks] = up_load16(rwdt, 32 * ks + kq < R ? off + 64u * ks : kUpDrop);
        }
    };
    // each wave's 16 x 64 delta tile goes through its own LDS slot (over the u tiles, unused
    // now) so that every store instruction writes whole 128-byte rows: lane l stores steps
    // 4 (l % 16) .. + 3 of channel rows l / 16, + 4, + 8, + 12
    constexpr int kSR = kUpTT + 8;  // slot row, in bf16
    uint16_t* slot = &s_u[0][0] + wave * 16 * kSR;
    auto dt_group = [&](int64_t g, const uint4 (&wf)[kUpGroup][KS]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kUpGroup; ++i) {
            const int64_t d0 = (wave + kW * (g * kUpGroup + i)) * 16;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                up_f32x4 o = up_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) o = up_mfma(up_frag(dtf[m][ks]), up_frag(wf[i][ks]), o);
                *reinterpret_cast<uint2*>(slot + (lane & 15) * kSR + 16 * m + trow) =
                    make_uint2(up_pack_bf16(o[0], o[1]), up_pack_bf16(o[2], o[3]));
            }
            __builtin_amdgcn_wave_barrier();  // the wave's LDS accesses run in order
            const int s4 = 4 * (lane & 15);
            const bool t_in = t0 + s4 < L;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = (lane >> 4) + 4 * j;
                const uint2 v = *reinterpret_cast<const uint2*>(slot + r * kSR + s4);
                const int64_t d = d0 + r;
                up_store8(rdl, (d < D && t_in) ? (uint32_t)((d * L + t0 + s4) * 2) : kUpDrop, v.x, v.y);
            }
            __builtin_amdgcn_wave_barrier();
        }
    };
    const int64_t ngroups = (dtiles + kW * kUpGroup - 1) / (kW * kUpGroup);  // the same for every wave
    uint4 wcur[kUpGroup][KS], wnext[kUpGroup][KS];
    wdt_fetch(0, wcur);
    for (int64_t g = 0; g < ngroups; ++g) {
        wdt_fetch(g + 1, wnext);  // before this group's stores: its wait never covers them
        __builtin_amdgcn_sched_barrier(0);
        dt_group(g, wcur);
#pragma unroll
        for (int i = 0; i < kUpGroup; ++i)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) wcur[i][ks] = wnext[i][ks];
    }
}

// ---------------------------------------------------------------------------------------------
// host side

// MAMBA_SCAN_ERR_UNSUPPORTED unless: len % 4 == 0, dim % 8 == 0 and <= kUpMaxDim,
// dt_rank % 8 == 0 and <= 64,
// dt_rank + 2 dstate <= 128, 1 <= d_conv <= 4, and the pointers aligned for the vector accesses.
template <int K>
int launch_upstream_k(const UpParams& q, int ks, hipStream_t stream) {
    const int64_t groups = q.batch * ((q.len + kUpTT - 1) / kUpTT);
    void* args[] = {const_cast<UpParams*>(&q)};
    const void* fn = ks == 1 ? reinterpret_cast<const void*>(&upstream_kernel<K, 1>)
                             : reinterpret_cast<const void*>(&upstream_kernel<K, 2>);
    return hipLaunchKernel(fn, dim3((unsigned)groups), dim3(kUpThreads), args, 0, stream) == hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

inline int launch_upstream(const UpParams& q, int d_conv, hipStream_t stream) {
    const int ks = q.dt_rank <= 32 ? 1 : 2;
    switch (d_conv) {
        case 1: return launch_upstream_k<1>(q, ks, stream);
        case 2: return launch_upstream_k<2>(q, ks, stream);
        case 3: return launch_upstream_k<3>(q, ks, stream);
        case 4: return launch_upstream_k<4>(q, ks, stream);
        default: return MAMBA_SCAN_ERR_UNSUPPORTED;
    }
}

}  // namespace mscan
