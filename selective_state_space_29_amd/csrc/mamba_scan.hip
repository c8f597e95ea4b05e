// C-ABI entry points of the selective-scan library: argument validation, kernel choice and the
// launch on the caller's stream. The contract is in include/mamba_scan.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "../../include/mamba_scan.h"
#include "block_upstream.hpp"  // UpParams and its limits (its kernel is built in k_upstream.hip)
#include "common.hpp"
#include "launch.hpp"
#include "bwd_layout.hpp"
#include "scan_lp.hpp"   // lp_eligible
#include "scan_ls.hpp"   // ls_eligible
#include "scan_step.hpp"  // step_eligible
#include "scan_tiled.hpp"  // aligned

#include <atomic>
#include <mutex>

using namespace mscan;

// flags the backward entry points take
constexpr uint32_t kBwdFlags =
    MAMBA_SCAN_DELTA_SOFTPLUS | MAMBA_SCAN_ZOH_B | MAMBA_SCAN_FORCE_TILED | MAMBA_SCAN_FORCE_LANES;

namespace {

struct Span {
    uintptr_t lo, hi;  // [lo, hi) bytes
    bool valid;
};

// Byte range touched by a tensor with the given sizes and element strides.
Span span_of(const void* ptr, int64_t esize, const int64_t* sizes, const int64_t* strides, int nd) {
    Span s{0, 0, false};
    if (!ptr) return s;
    int64_t maxoff = 0;
    for (int i = 0; i < nd; ++i) {
        if (sizes[i] <= 0) return s;  // no elements: nothing is read or written
        maxoff += (sizes[i] - 1) * strides[i];
    }
    s.lo = reinterpret_cast<uintptr_t>(ptr);
    s.hi = s.lo + (uintptr_t)((maxoff + 1) * esize);
    s.valid = true;
    return s;
}

const int64_t kUnit[1] = {1};

bool overlaps(const Span& a, const Span& b) { return a.valid && b.valid && a.lo < b.hi && b.lo < a.hi; }

void contiguous_strides(const mamba_scan_shape& s, mamba_scan_strides* st) {
    const int64_t DL = s.dim * s.len, NL = s.dstate * s.len, DN = s.dim * s.dstate;
    const int64_t t3[3] = {DL, s.len, 1};
    memcpy(st->u, t3, sizeof t3);
    memcpy(st->delta, t3, sizeof t3);
    memcpy(st->z, t3, sizeof t3);
    memcpy(st->y, t3, sizeof t3);
    const int64_t bc[3] = {NL, s.len, 1};
    memcpy(st->B, bc, sizeof bc);
    memcpy(st->C, bc, sizeof bc);
    const int64_t hs[3] = {DN, s.dstate, 1};
    memcpy(st->h0, hs, sizeof hs);
    memcpy(st->last_state, hs, sizeof hs);
    st->A[0] = s.dstate;
    st->A[1] = 1;
    st->D = 1;
    st->delta_bias = 1;
}

// batch, dim and len may be 0 (an empty call); dstate must be at least 1.
bool bad_shape(const mamba_scan_shape& s) { return s.batch < 0 || s.dim < 0 || s.len < 0 || s.dstate <= 0; }

// What an empty call does: 0 = not empty; 1 = nothing (no (batch, channel) row, or no step and no
// last_state); 2 = no step, last_state written with h0 or zeros (the generic kernel, whose step
// loop then runs no iteration).
int empty_plan(const mamba_scan_shape& s, uint32_t flags) {
    if (s.batch * s.dim == 0) return 1;
    if (s.len == 0) return (flags & MAMBA_SCAN_RETURN_LAST_STATE) ? 2 : 1;
    return 0;
}

int validate(const mamba_scan_ptrs* p, const mamba_scan_shape* s, const mamba_scan_strides* st,
             mamba_scan_dtype dtype, uint32_t flags) {
    if (!p || !s || !st) return MAMBA_SCAN_ERR_NULL;
    if (dtype != MAMBA_SCAN_F32 && dtype != MAMBA_SCAN_BF16) return MAMBA_SCAN_ERR_DTYPE;
    if (flags & ~MAMBA_SCAN_KNOWN_FLAGS) return MAMBA_SCAN_ERR_ARGS;
    const uint32_t forced = flags & (MAMBA_SCAN_FORCE_GENERIC | MAMBA_SCAN_FORCE_TILED | MAMBA_SCAN_FORCE_LANES |
                                     MAMBA_SCAN_FORCE_CHUNKED | MAMBA_SCAN_FORCE_STEP);
    if (forced & (forced - 1)) return MAMBA_SCAN_ERR_ARGS;  // at most one kernel may be forced
    if (bad_shape(*s)) return MAMBA_SCAN_ERR_SHAPE;
    if (s->dstate > MAMBA_SCAN_MAX_DSTATE) return MAMBA_SCAN_ERR_DSTATE;
    // a tensor with no elements is never touched: its pointer may be NULL
    const bool rows = s->batch * s->dim > 0, steps = s->batch * s->len > 0;
    if ((rows && s->len > 0 && (!p->u || !p->delta || !p->y)) || (steps && (!p->B || !p->C)) ||
        (s->dim > 0 && !p->A))
        return MAMBA_SCAN_ERR_NULL;
    const bool want_ls = (flags & MAMBA_SCAN_RETURN_LAST_STATE) != 0;
    if (want_ls ? (rows && !p->last_state) : p->last_state != nullptr) return MAMBA_SCAN_ERR_ARGS;
    if (p->workspace_bytes < 0 || (p->workspace_bytes > 0 && !p->workspace)) return MAMBA_SCAN_ERR_ARGS;

    const int64_t* inner3[] = {st->u, st->delta, st->z, st->B, st->C, st->y, st->h0, st->last_state};
    for (const int64_t* v : inner3) {
        if (v[2] != 1) return MAMBA_SCAN_ERR_STRIDE;
        if (v[0] < 0 || v[1] < 0) return MAMBA_SCAN_ERR_SHAPE;
    }
    if (st->A[1] != 1) return MAMBA_SCAN_ERR_STRIDE;
    if (st->A[0] < 0 || st->D < 0 || st->delta_bias < 0) return MAMBA_SCAN_ERR_SHAPE;

    // Outputs may not overlap inputs or each other.
    const int64_t es = dtype == MAMBA_SCAN_BF16 ? 2 : 4;
    const int64_t bdl[3] = {s->batch, s->dim, s->len};
    const int64_t bnl[3] = {s->batch, s->dstate, s->len};
    const int64_t bdn[3] = {s->batch, s->dim, s->dstate};
    const int64_t dn[2] = {s->dim, s->dstate};
    const int64_t d1[1] = {s->dim};
    const Span ins[] = {
        span_of(p->u, es, bdl, st->u, 3),         span_of(p->delta, es, bdl, st->delta, 3),
        span_of(p->z, es, bdl, st->z, 3),         span_of(p->B, es, bnl, st->B, 3),
        span_of(p->C, es, bnl, st->C, 3),         span_of(p->A, 4, dn, st->A, 2),
        span_of(p->D, 4, d1, &st->D, 1),          span_of(p->delta_bias, 4, d1, &st->delta_bias, 1),
        span_of(p->h0, 4, bdn, st->h0, 3),
        span_of(p->workspace, 1, &p->workspace_bytes, kUnit, p->workspace_bytes > 0 ? 1 : 0),
    };
    const Span y = span_of(p->y, 4, bdl, st->y, 3);
    const Span ls = span_of(p->last_state, 4, bdn, st->last_state, 3);
    for (const Span& in : ins)
        if (overlaps(y, in) || overlaps(ls, in)) return MAMBA_SCAN_ERR_ARGS;
    if (overlaps(y, ls)) return MAMBA_SCAN_ERR_ARGS;
    // with SAVE_CHECKPOINTS the workspace is written: it may not overlap any input either
    if (flags & MAMBA_SCAN_SAVE_CHECKPOINTS) {
        const Span& ws = ins[sizeof ins / sizeof ins[0] - 1];
        for (size_t i = 0; i + 1 < sizeof ins / sizeof ins[0]; ++i)
            if (overlaps(ws, ins[i])) return MAMBA_SCAN_ERR_ARGS;
    }
    return MAMBA_SCAN_OK;
}

ScanParams make_params(const mamba_scan_ptrs* p, const mamba_scan_shape* s, const mamba_scan_strides* st,
                       uint32_t flags) {
    ScanParams q;
    q.u = p->u;
    q.delta = p->delta;
    q.z = p->z;
    q.B = p->B;
    q.C = p->C;
    q.A = p->A;
    q.D = p->D;
    q.bias = p->delta_bias;
    q.h0 = p->h0;
    q.y = p->y;
    q.zoh_b = (flags & MAMBA_SCAN_ZOH_B) ? 1 : 0;
    q.last_state = (flags & MAMBA_SCAN_RETURN_LAST_STATE) ? p->last_state : nullptr;
    q.batch = s->batch;
    q.dim = s->dim;
    q.len = s->len;
    q.dstate = s->dstate;
    q.su_b = st->u[0];
    q.su_d = st->u[1];
    q.sdt_b = st->delta[0];
    q.sdt_d = st->delta[1];
    q.sz_b = st->z[0];
    q.sz_d = st->z[1];
    q.sB_b = st->B[0];
    q.sB_n = st->B[1];
    q.sC_b = st->C[0];
    q.sC_n = st->C[1];
    q.sy_b = st->y[0];
    q.sy_d = st->y[1];
    q.sh0_b = st->h0[0];
    q.sh0_d = st->h0[1];
    q.sls_b = st->last_state[0];
    q.sls_d = st->last_state[1];
    q.sA_d = st->A[0];
    q.sD = st->D;
    q.sbias = st->delta_bias;
    q.softplus = (flags & MAMBA_SCAN_DELTA_SOFTPLUS) ? 1 : 0;
    q.ck = (flags & MAMBA_SCAN_SAVE_CHECKPOINTS) ? static_cast<float*>(p->workspace) : nullptr;
    q.ck_nseg = (s->len + 15) / 16;
    return q;
}

// Compute units of the current device (cached per device; 0 if the runtime cannot say).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev < 0 || dev >= 64) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// The chunked kernel is the default for sequences of at least kChunkedMinLen steps where the
// lane-per-state kernel (4 channels x 16 states per wave) would give the GPU's SIMDs fewer than
// two waves each. (Shorter calls, such as the pieces of a streamed sequence, keep the sequential
// kernel, whose results do not depend on where a sequence is split.)
constexpr int64_t kChunkedMinLen = 1024;
bool prefer_chunked(const ScanParams& q) {
    if (q.dstate != 16 || q.len < kChunkedMinLen) return false;
    const int cus = device_cus();
    if (cus <= 0) return false;
    const int64_t ls_waves = q.batch * ((q.dim + 3) / 4);
    return ls_waves < 2 * 4 * (int64_t)cus;
}

// With SAVE_CHECKPOINTS the states go to the workspace: it must hold them, 4-byte aligned.
int check_checkpoint_workspace(const mamba_scan_ptrs* p, const mamba_scan_shape* s, uint32_t flags) {
    if (!(flags & MAMBA_SCAN_SAVE_CHECKPOINTS)) return MAMBA_SCAN_OK;
    const int64_t need = s->batch * s->dim * ((s->len + 15) / 16) * s->dstate * 4;
    if (need == 0) return MAMBA_SCAN_OK;  // an empty call saves nothing
    if (!p->workspace || p->workspace_bytes < need) return MAMBA_SCAN_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(p->workspace) % 4) return MAMBA_SCAN_ERR_ARGS;
    return MAMBA_SCAN_OK;
}

// The forward kernel a call runs: a forced one if it can take the case, else the default order.
// Shared by mamba_scan_fwd and mamba_scan_fwd_kernel so that the query and the launch agree.
int choose_kernel(const ScanParams& q, uint32_t flags, bool bf16) {
    const int64_t es = bf16 ? 2 : 4;
    if (q.ck) {  // the saved states come from the lane-per-state and chunked kernels only
        if (flags & (MAMBA_SCAN_FORCE_GENERIC | MAMBA_SCAN_FORCE_TILED | MAMBA_SCAN_FORCE_STEP))
            return MAMBA_SCAN_ERR_UNSUPPORTED;
        if (flags & MAMBA_SCAN_FORCE_CHUNKED) return lp_eligible(q, es) ? MAMBA_SCAN_KERNEL_CHUNKED : MAMBA_SCAN_ERR_UNSUPPORTED;
        if (!(flags & MAMBA_SCAN_FORCE_LANES) && prefer_chunked(q) && lp_eligible(q, es)) return MAMBA_SCAN_KERNEL_CHUNKED;
        return ls_eligible(q, es) ? MAMBA_SCAN_KERNEL_LANES : MAMBA_SCAN_ERR_UNSUPPORTED;
    }
    if (flags & MAMBA_SCAN_FORCE_STEP) return step_eligible(q) ? MAMBA_SCAN_KERNEL_STEP : MAMBA_SCAN_ERR_UNSUPPORTED;
    if (flags & MAMBA_SCAN_FORCE_CHUNKED) return lp_eligible(q, es) ? MAMBA_SCAN_KERNEL_CHUNKED : MAMBA_SCAN_ERR_UNSUPPORTED;
    if (flags & MAMBA_SCAN_FORCE_LANES) return ls_eligible(q, es) ? MAMBA_SCAN_KERNEL_LANES : MAMBA_SCAN_ERR_UNSUPPORTED;
    if (flags & MAMBA_SCAN_FORCE_TILED) return tiled_can_run_any(q, bf16) ? MAMBA_SCAN_KERNEL_TILED : MAMBA_SCAN_ERR_UNSUPPORTED;
    if (flags & MAMBA_SCAN_FORCE_GENERIC) return MAMBA_SCAN_KERNEL_GENERIC;
    if (q.len <= kStepMaxLen && step_eligible(q)) return MAMBA_SCAN_KERNEL_STEP;
    if (prefer_chunked(q) && lp_eligible(q, es)) return MAMBA_SCAN_KERNEL_CHUNKED;
    if (ls_eligible(q, es)) return MAMBA_SCAN_KERNEL_LANES;
    if (tiled_can_run_any(q, bf16)) return MAMBA_SCAN_KERNEL_TILED;
    return MAMBA_SCAN_KERNEL_GENERIC;
}

int backward_entry(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape* s, mamba_scan_dtype dtype,
                   uint32_t flags, void* stream);

}  // namespace

namespace mscan {

// The forward launch that writes the saved states when the backward recomputes them: the kernel
// that a forward call with SAVE_CHECKPOINTS runs by default (chunked or lane-per-state), so that
// the backward's states are those bits either way.
int launch_fwd_checkpoints(const ScanParams& q, bool bf16, hipStream_t stream) {
    const int k = choose_kernel(q, 0, bf16);
    if (k == MAMBA_SCAN_KERNEL_CHUNKED) return launch_lp_any(q, bf16, stream);
    if (k == MAMBA_SCAN_KERNEL_LANES) return launch_ls_any(q, bf16, stream);
    return k < 0 ? k : MAMBA_SCAN_ERR_UNSUPPORTED;
}

}  // namespace mscan


// The static workspace of mamba_scan_bwd_static: every GPU the library runs on holds its own copy
// until the process ends. In host code this name is only a handle for hipGetSymbolAddress; the
// device address it resolves to, per device, is what kernels and copies are given.
static __device__ __align__(256) unsigned char scratch[MAMBA_SCAN_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    int rc = MAMBA_SCAN_OK;
};
ScratchSlot g_scratch[kMaxDevices];

// The device address of the current device's scratch, looked up once per device (with that
// device current) on the first call that needs it.
int device_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MAMBA_SCAN_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return MAMBA_SCAN_ERR_UNSUPPORTED;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            slot.rc = MAMBA_SCAN_ERR_LAUNCH;
            return;
        }
        slot.ptr = ptr;
    });
    if (slot.rc != MAMBA_SCAN_OK) return slot.rc;
    *out = slot.ptr;
    return MAMBA_SCAN_OK;
}

}  // namespace

extern "C" {

int mamba_scan_abi_version(void) { return MAMBA_SCAN_ABI_VERSION; }

const char* mamba_scan_strerror(int code) {
    switch (code) {
        case MAMBA_SCAN_OK: return "success";
        case MAMBA_SCAN_ERR_NULL: return "a required pointer is NULL";
        case MAMBA_SCAN_ERR_SHAPE: return "a dimension is negative, dstate < 1, or a stride is negative";
        case MAMBA_SCAN_ERR_STRIDE: return "an innermost stride (along len, or along dstate) is not 1";
        case MAMBA_SCAN_ERR_DTYPE: return "unknown dtype (expected MAMBA_SCAN_F32 or MAMBA_SCAN_BF16)";
        case MAMBA_SCAN_ERR_DSTATE: return "dstate exceeds MAMBA_SCAN_MAX_DSTATE";
        case MAMBA_SCAN_ERR_ARGS:
            return "inconsistent flags/pointers (unknown flag, last_state vs RETURN_LAST_STATE, "
                   "workspace) or overlapping buffers";
        case MAMBA_SCAN_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
        case MAMBA_SCAN_ERR_UNSUPPORTED: return "the forced kernel cannot handle this shape or alignment";
        case MAMBA_SCAN_ERR_WORKSPACE: return "workspace too small";
        case MAMBA_SCAN_ERR_SCRATCH:
            return "the call needs more workspace than the static scratch buffer holds "
                   "(MAMBA_SCAN_STATIC_SCRATCH_BYTES)";
        default: return "unknown error code";
    }
}

int64_t mamba_scan_workspace_bytes(const mamba_scan_shape* s, mamba_scan_dtype dtype, uint32_t flags) {
    if (!s) return MAMBA_SCAN_ERR_NULL;
    if (dtype != MAMBA_SCAN_F32 && dtype != MAMBA_SCAN_BF16) return MAMBA_SCAN_ERR_DTYPE;
    if (flags & ~MAMBA_SCAN_KNOWN_FLAGS) return MAMBA_SCAN_ERR_ARGS;
    if (bad_shape(*s)) return MAMBA_SCAN_ERR_SHAPE;
    if (s->dstate > MAMBA_SCAN_MAX_DSTATE) return MAMBA_SCAN_ERR_DSTATE;
    if (flags & MAMBA_SCAN_SAVE_CHECKPOINTS) return s->batch * s->dim * ((s->len + 15) / 16) * s->dstate * 4;
    return 0;
}

int64_t mamba_scan_bwd_workspace_bytes(const mamba_scan_shape* s, mamba_scan_dtype dtype, uint32_t flags) {
    if (!s) return MAMBA_SCAN_ERR_NULL;
    if (dtype != MAMBA_SCAN_F32 && dtype != MAMBA_SCAN_BF16) return MAMBA_SCAN_ERR_DTYPE;
    if (flags & ~(kBwdFlags | MAMBA_SCAN_SAVE_CHECKPOINTS)) return MAMBA_SCAN_ERR_ARGS;
    if (bad_shape(*s)) return MAMBA_SCAN_ERR_SHAPE;
    if (s->dstate > MAMBA_SCAN_MAX_DSTATE) return MAMBA_SCAN_ERR_DSTATE;
    if ((flags & MAMBA_SCAN_FORCE_LANES) && (flags & MAMBA_SCAN_FORCE_TILED)) return MAMBA_SCAN_ERR_ARGS;
    if (s->batch * s->dim * s->len == 0) return 0;  // an empty call runs no scan
    const int pick = bwd_pick(*s, dtype == MAMBA_SCAN_BF16 ? 2 : 4, flags);
    if (pick < 0) return pick;
    const bool given_ck = (flags & MAMBA_SCAN_SAVE_CHECKPOINTS) != 0;
    return pick ? bwd_ls_layout(*s, given_ck).total : bwd_layout(*s, given_ck).total;
}

int mamba_scan_bwd(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape* s, mamba_scan_dtype dtype,
                   uint32_t flags, void* stream) {
    return backward_entry(p, s, dtype, flags, stream);
}

int mamba_scan_bwd_static(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape* s, mamba_scan_dtype dtype,
                          uint32_t flags, void* stream) {
    if (!p || !s) return MAMBA_SCAN_ERR_NULL;
    if (p->workspace || p->workspace_bytes != 0) return MAMBA_SCAN_ERR_ARGS;  // the scratch is the library's
    if (flags & ~kBwdFlags) return MAMBA_SCAN_ERR_ARGS;
    const int64_t need =
        mamba_scan_bwd_workspace_bytes(s, dtype, flags | (p->checkpoints ? MAMBA_SCAN_SAVE_CHECKPOINTS : 0u));
    if (need < 0) return (int)need;
    if (need > MAMBA_SCAN_STATIC_SCRATCH_BYTES) return MAMBA_SCAN_ERR_SCRATCH;
    void* ws = nullptr;
    const int rc = device_scratch(&ws);
    if (rc != MAMBA_SCAN_OK) return rc;
    mamba_scan_bwd_ptrs q = *p;
    q.workspace = ws;
    q.workspace_bytes = MAMBA_SCAN_STATIC_SCRATCH_BYTES;
    return backward_entry(&q, s, dtype, flags, stream);
}

}  // extern "C"

namespace {

int backward_entry(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape* s, mamba_scan_dtype dtype,
                   uint32_t flags, void* stream) {
    if (!p || !s) return MAMBA_SCAN_ERR_NULL;
    if (flags & ~kBwdFlags) return MAMBA_SCAN_ERR_ARGS;
    const int64_t need =
        mamba_scan_bwd_workspace_bytes(s, dtype, flags | (p->checkpoints ? MAMBA_SCAN_SAVE_CHECKPOINTS : 0u));
    if (need < 0) return (int)need;
    // pointers of tensors with elements (batch, dim and len may be 0: an empty call)
    const bool cells = s->batch * s->dim * s->len > 0, steps = s->batch * s->len > 0;
    if ((cells && (!p->u || !p->delta || !p->dy || !p->du || !p->ddelta)) ||
        (steps && (!p->B || !p->C || !p->dB || !p->dC)) || (s->dim > 0 && (!p->A || !p->dA)))
        return MAMBA_SCAN_ERR_NULL;
    if ((cells && (p->z != nullptr) != (p->dz != nullptr)) ||
        (s->dim > 0 && ((p->D != nullptr) != (p->dD != nullptr) ||
                        (p->delta_bias != nullptr) != (p->ddelta_bias != nullptr))))
        return MAMBA_SCAN_ERR_ARGS;
    if (p->workspace_bytes < 0 || (p->workspace_bytes > 0 && !p->workspace)) return MAMBA_SCAN_ERR_ARGS;
    if (need > 0 && (!p->workspace || p->workspace_bytes < need)) return MAMBA_SCAN_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(p->workspace) % 256 != 0) return MAMBA_SCAN_ERR_ARGS;
    if (reinterpret_cast<uintptr_t>(p->checkpoints) % 4 != 0) return MAMBA_SCAN_ERR_ARGS;
    const int64_t es = dtype == MAMBA_SCAN_BF16 ? 2 : 4;
    const bool lanes = bwd_pick(*s, es, flags) == 1;  // an error was returned by the size query
    if (!lanes && s->batch * ((s->dim + 63) / 64) > 0x7fffffff) return MAMBA_SCAN_ERR_UNSUPPORTED;

    const int64_t DL = s->batch * s->dim * s->len, NL = s->batch * s->dstate * s->len;
    const int64_t DN = s->batch * s->dim * s->dstate;
    auto span = [](const void* ptr, int64_t bytes) {
        Span x{0, 0, false};
        if (!ptr || bytes <= 0) return x;  // no elements: nothing is read or written
        x.lo = reinterpret_cast<uintptr_t>(ptr);
        x.hi = x.lo + (uintptr_t)bytes;
        x.valid = true;
        return x;
    };
    const Span ins[] = {span(p->u, DL * es), span(p->delta, DL * es), span(p->z, DL * es), span(p->B, NL * es),
                        span(p->C, NL * es), span(p->A, s->dim * s->dstate * 4), span(p->D, s->dim * 4),
                        span(p->delta_bias, s->dim * 4), span(p->h0, DN * 4), span(p->dy, DL * 4),
                        span(p->dlast_state, DN * 4), span(p->workspace, p->workspace_bytes),
                        span(p->checkpoints, s->batch * s->dim * ((s->len + 15) / 16) * s->dstate * 4)};
    const Span outs[] = {span(p->du, DL * 4), span(p->ddelta, DL * 4), span(p->dz, DL * 4),
                         span(p->dB, NL * 4), span(p->dC, NL * 4), span(p->dA, s->dim * s->dstate * 4),
                         span(p->dD, s->dim * 4), span(p->ddelta_bias, s->dim * 4), span(p->dh0, DN * 4)};
    for (const Span& o : outs) {
        for (const Span& i : ins)
            if (overlaps(o, i)) return MAMBA_SCAN_ERR_ARGS;
        for (const Span& o2 : outs)
            if (&o2 != &o && overlaps(o, o2)) return MAMBA_SCAN_ERR_ARGS;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (!cells) {
        // no scan: the gradients that have elements are sums over nothing, except that of the
        // initial state over no steps, which is the final state's (or zero)
        int rc = MAMBA_SCAN_OK;
        auto fill = [&](float* dst, const float* src, int64_t n) {
            if (rc == MAMBA_SCAN_OK) rc = launch_bwd_fill(dst, src, n, hs);
        };
        fill(p->dA, nullptr, s->dim * s->dstate);
        fill(p->dD, nullptr, s->dim);
        fill(p->ddelta_bias, nullptr, s->dim);
        fill(p->dB, nullptr, NL);
        fill(p->dC, nullptr, NL);
        fill(p->dh0, s->len == 0 ? p->dlast_state : nullptr, DN);
        return rc;
    }
    const bool sp = (flags & MAMBA_SCAN_DELTA_SOFTPLUS) != 0;
    if (flags & MAMBA_SCAN_ZOH_B)
        return lanes ? launch_bwd_ls_zoh_any(p, *s, dtype == MAMBA_SCAN_BF16, sp, hs)
                     : launch_bwd_tiled_zoh_any(p, *s, dtype == MAMBA_SCAN_BF16, sp, hs);
    return lanes ? launch_bwd_ls_any(p, *s, dtype == MAMBA_SCAN_BF16, sp, hs)
                 : launch_bwd_tiled_any(p, *s, dtype == MAMBA_SCAN_BF16, sp, hs);
}

}  // namespace

extern "C" {

int mamba_block_upstream(const mamba_upstream_ptrs* p, const mamba_upstream_shape* s, mamba_scan_dtype dtype,
                         void* stream) {
    if (!p || !s) return MAMBA_SCAN_ERR_NULL;
    if (!p->x || !p->conv_w || !p->w_x || !p->w_dt || !p->u || !p->xdbl || !p->delta) return MAMBA_SCAN_ERR_NULL;
    if (s->batch <= 0 || s->dim <= 0 || s->len <= 0 || s->dstate <= 0 || s->dt_rank <= 0 || s->d_conv <= 0)
        return MAMBA_SCAN_ERR_SHAPE;
    if (dtype != MAMBA_SCAN_BF16) return dtype == MAMBA_SCAN_F32 ? MAMBA_SCAN_ERR_UNSUPPORTED : MAMBA_SCAN_ERR_DTYPE;
    const int64_t J = s->dt_rank + 2 * s->dstate;
    if (s->len % 4 || s->dim % 8 || s->dim > kUpMaxDim || s->dt_rank % 8 || s->dt_rank > 64 || J > 128 || s->d_conv > 4)
        return MAMBA_SCAN_ERR_UNSUPPORTED;
    if (!aligned(p->x, 8) || !aligned(p->u, 8) || !aligned(p->delta, 8) || !aligned(p->xdbl, 8) ||
        !aligned(p->w_x, 16) || !aligned(p->w_dt, 16) || !aligned(p->conv_w, 4) ||
        (p->conv_b && !aligned(p->conv_b, 4)))
        return MAMBA_SCAN_ERR_UNSUPPORTED;
    if (s->batch * ((s->len + kUpTT - 1) / kUpTT) > 0x7fffffff) return MAMBA_SCAN_ERR_UNSUPPORTED;
    // one batch of each tensor is addressed with 32-bit byte offsets
    if (s->dim * s->len * 2 >= ((int64_t)1 << 31) || J * s->len * 2 >= ((int64_t)1 << 31))
        return MAMBA_SCAN_ERR_UNSUPPORTED;
    const int64_t DL = s->batch * s->dim * s->len;
    auto span = [](const void* ptr, int64_t bytes) {
        Span x{0, 0, false};
        if (!ptr) return x;
        x.lo = reinterpret_cast<uintptr_t>(ptr);
        x.hi = x.lo + (uintptr_t)bytes;
        x.valid = true;
        return x;
    };
    const Span ins[] = {span(p->x, DL * 2), span(p->conv_w, s->dim * s->d_conv * 4), span(p->conv_b, s->dim * 4),
                        span(p->w_x, J * s->dim * 2), span(p->w_dt, s->dim * s->dt_rank * 2)};
    const Span outs[] = {span(p->u, DL * 2), span(p->xdbl, s->batch * J * s->len * 2), span(p->delta, DL * 2)};
    for (const Span& o : outs) {
        for (const Span& i : ins)
            if (overlaps(o, i)) return MAMBA_SCAN_ERR_ARGS;
        for (const Span& o2 : outs)
            if (&o2 != &o && overlaps(o, o2)) return MAMBA_SCAN_ERR_ARGS;
    }
    UpParams q;
    q.x = static_cast<const uint16_t*>(p->x);
    q.conv_w = p->conv_w;
    q.conv_b = p->conv_b;
    q.w_x = static_cast<const uint16_t*>(p->w_x);
    q.w_dt = static_cast<const uint16_t*>(p->w_dt);
    q.u = static_cast<uint16_t*>(p->u);
    q.xdbl = static_cast<uint16_t*>(p->xdbl);
    q.delta = static_cast<uint16_t*>(p->delta);
    q.batch = s->batch;
    q.dim = s->dim;
    q.len = s->len;
    q.dstate = (int)s->dstate;
    q.dt_rank = (int)s->dt_rank;
    return launch_upstream_any(q, (int)s->d_conv, static_cast<hipStream_t>(stream));
}

int mamba_scan_fwd(const mamba_scan_ptrs* p, const mamba_scan_shape* s, const mamba_scan_strides* st_in,
                   mamba_scan_dtype dtype, uint32_t flags, void* stream) {
    if (!p || !s) return MAMBA_SCAN_ERR_NULL;
    mamba_scan_strides st;
    if (st_in) {
        st = *st_in;
    } else {
        if (bad_shape(*s)) return MAMBA_SCAN_ERR_SHAPE;
        contiguous_strides(*s, &st);
    }
    const int rc = validate(p, s, &st, dtype, flags);
    if (rc != MAMBA_SCAN_OK) return rc;
    const ScanParams q = make_params(p, s, &st, flags);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool bf16 = dtype == MAMBA_SCAN_BF16;

    const int wrc = check_checkpoint_workspace(p, s, flags);
    if (wrc != MAMBA_SCAN_OK) return wrc;
    if (const int e = empty_plan(*s, flags)) return e == 1 ? MAMBA_SCAN_OK : launch_generic_any(q, bf16, hs);
    const int kernel = choose_kernel(q, flags, bf16);
    switch (kernel) {
        case MAMBA_SCAN_KERNEL_CHUNKED: return launch_lp_any(q, bf16, hs);
        case MAMBA_SCAN_KERNEL_STEP: return launch_step_any(q, bf16, hs);
        case MAMBA_SCAN_KERNEL_LANES: return launch_ls_any(q, bf16, hs);
        case MAMBA_SCAN_KERNEL_TILED: return launch_tiled_any(q, bf16, hs);
        case MAMBA_SCAN_KERNEL_GENERIC: return launch_generic_any(q, bf16, hs);
        default: return kernel;  // an error code
    }
}

int mamba_scan_fwd_kernel(const mamba_scan_ptrs* p, const mamba_scan_shape* s, const mamba_scan_strides* st_in,
                          mamba_scan_dtype dtype, uint32_t flags) {
    if (!p || !s) return MAMBA_SCAN_ERR_NULL;
    mamba_scan_strides st;
    if (st_in) {
        st = *st_in;
    } else {
        if (bad_shape(*s)) return MAMBA_SCAN_ERR_SHAPE;
        contiguous_strides(*s, &st);
    }
    const int rc = validate(p, s, &st, dtype, flags);
    if (rc != MAMBA_SCAN_OK) return rc;
    const int wrc = check_checkpoint_workspace(p, s, flags);
    if (wrc != MAMBA_SCAN_OK) return wrc;
    if (const int e = empty_plan(*s, flags)) return e == 1 ? MAMBA_SCAN_KERNEL_NONE : MAMBA_SCAN_KERNEL_GENERIC;
    const ScanParams q = make_params(p, s, &st, flags);
    return choose_kernel(q, flags, dtype == MAMBA_SCAN_BF16);
}

}  // extern "C"
