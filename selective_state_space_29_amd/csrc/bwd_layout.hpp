// Workspace layouts of the backward pass (host side), shared by its launchers and the C-ABI entry
// points that size and check the caller's workspace, and the choice between its two kernels.
#pragma once

#include <stdint.h>

#include "../../include/mamba_scan.h"

namespace mscan {

constexpr int kBwdSeg = 16;  // steps per segment (checkpoint interval)

struct BwdLayout {
    int64_t lp, nseg, groups;
    // lane-per-state kernel: sequence parts and segments per part; the pre-pass's sub-parts
    // (kBlsSub per part) and segments per sub-part
    int64_t parts = 1, spp = 0, subs = 1, sspp = 0;
    int64_t off_bc, off_ck, off_bcpart, off_apart, off_dpart, off_bpart, off_carry = 0, total;
};

inline int64_t bwd_align(int64_t x) { return (x + 255) / 256 * 256; }

// States per launch: blocks of 16; a remainder in (8, 16] that is odd (two states per wave would
// leave one wave half used) is split into 8 and the rest.
inline int64_t bwd_next_block(int64_t rem) { return rem > 16 ? 16 : (rem > 8 && rem % 2) ? 8 : rem; }
inline int64_t bwd_block_states(int64_t N) { return bwd_next_block(N); }

// given_ck: the caller passes the forward's saved states, so no region for recomputed ones
inline BwdLayout bwd_layout(const mamba_scan_shape& s, bool given_ck = false) {
    BwdLayout l;
    l.lp = (s.len + kBwdSeg - 1) / kBwdSeg * kBwdSeg;
    l.nseg = l.lp / kBwdSeg;
    l.groups = (s.dim + 63) / 64;
    int64_t o = 0;
    l.off_bc = o;
    o = bwd_align(o + 2 * s.batch * s.dstate * l.lp * 4);
    l.off_ck = o;
    if (!given_ck) o = bwd_align(o + s.batch * s.dim * l.nseg * bwd_block_states(s.dstate) * 4);
    l.off_bcpart = o;
    o = bwd_align(o + l.groups * s.batch * 2 * s.dstate * l.lp * 4);
    l.off_apart = o;
    o = bwd_align(o + s.batch * s.dim * s.dstate * 4);
    l.off_dpart = o;
    o = bwd_align(o + s.batch * s.dim * 4);
    l.off_bpart = o;
    o = bwd_align(o + s.batch * s.dim * 4);
    l.total = o;
    return l;
}

// The fixed-order reduction that finishes both backward kernels: dB, dC over the channel groups'
// partials, dA, dD, dbias over the sequence parts and the batch.
struct BwdReduceParams {
    const float* bcpart;
    const float* apart;  // (parts, batch, dim, dstate)
    const float* dpart;  // (parts, batch, dim)
    const float* bpart;
    float* dB;
    float* dC;
    float* dA;
    float* dD;
    float* dbias;
    int64_t batch, dim, len, dstate, lp, groups;
    int64_t parts = 1;
};

// Lane-per-state backward (16, 32, 64 states): workgroups of kBlsW waves, 4 channels per wave. Four waves:
// a SIMD's 3 waves then belong to 3 workgroups, whose barriers do not wait together (measured at
// the Mamba-130m shape: 518 us per launch against 637 us with 6-wave workgroups, whose smaller
// dB / dC partials did not make up for it).
constexpr int kBlsW = 4;

// 16, 32 or 64 states (the state counts the forward lane-per-state kernels save states for), and
// byte offsets that fit 31 bits: a wave's 4 fp32 rows, a batch's B / C, a wave's saved states
// (the forward lane-per-state kernel that writes them has the same limits).
inline bool bwd_ls_fits(const mamba_scan_shape& s, int64_t es) {
    const int64_t N = s.dstate;
    if (N != 16 && N != 32 && N != 64) return false;
    const int64_t lim = (int64_t)1 << 31;
    const int64_t nseg = (s.len + kBwdSeg - 1) / kBwdSeg;
    if (4 * s.len * 4 >= lim || N * s.len * es >= lim || 4 * nseg * N * 4 >= lim) return false;
    return s.batch * s.dim <= 0x7fffffff;
}

// 1: the lane-per-state kernel, 0: the segment-tiled one, < 0: an error code. By default the
// lane-per-state kernel wherever it can run.
inline int bwd_pick(const mamba_scan_shape& s, int64_t es, uint32_t flags) {
    const bool fl = (flags & MAMBA_SCAN_FORCE_LANES) != 0, ft = (flags & MAMBA_SCAN_FORCE_TILED) != 0;
    if (fl && ft) return MAMBA_SCAN_ERR_ARGS;
    if (ft) return 0;
    const bool ok = bwd_ls_fits(s, es);
    if (fl && !ok) return MAMBA_SCAN_ERR_UNSUPPORTED;
    return ok ? 1 : 0;
}

// Sequence parts of the lane-per-state backward: where the (batch, channel) rows give fewer than
// kBlsWaveTarget waves (3 per SIMD of a 256-CU GPU), the segments are split into up to
// kBlsMaxParts parts of at least kBlsMinSegs segments (512 steps: the split costs a launch and
// about 15 us at the mamba-minimal shape, 16 segments, where it lost 59 against 44 us) that run
// side by side, each part's reverse
// starting from the adjoint that the later parts hand it (a pre-pass computes each part's own
// contribution and decay product). A function of the shape alone, so that the workspace size does
// not depend on the device.
constexpr int64_t kBlsWaveTarget = 3 * 4 * 256;
constexpr int64_t kBlsMaxParts = 64;
constexpr int64_t kBlsMinSegs = 32;
// The pre-pass runs each part as kBlsSub sub-parts, one wave per 4 channels each, so that its
// waves (one state chain per lane, a few instructions per step) fill the SIMDs four times as
// deep (at the genomic shape 8 waves per SIMD: 8.99 against 9.32 ms per backward call with 2).
constexpr int64_t kBlsSub = 4;
inline int64_t bwd_ls_parts(const mamba_scan_shape& s, int64_t nseg, int64_t groups) {
    const int64_t waves = s.batch * groups * kBlsW;
    int64_t P = (kBlsWaveTarget + waves - 1) / waves;
    const int64_t by_len = nseg / kBlsMinSegs > 1 ? nseg / kBlsMinSegs : 1;
    if (P > by_len) P = by_len;
    if (P > kBlsMaxParts) P = kBlsMaxParts;
    return P < 1 ? 1 : P;
}

// The lane-per-state kernel's workspace: the recomputed states (unless given), the dB / dC
// partials of its channel groups (4 kBlsW channels each), the dA / dD / dbias partials of every
// sequence part, and each later part's adjoint contribution and decay product.
inline BwdLayout bwd_ls_layout(const mamba_scan_shape& s, bool given_ck = false) {
    BwdLayout l;
    l.lp = (s.len + kBwdSeg - 1) / kBwdSeg * kBwdSeg;
    l.nseg = l.lp / kBwdSeg;
    l.groups = (s.dim + 4 * kBlsW - 1) / (4 * kBlsW);
    l.parts = bwd_ls_parts(s, l.nseg, l.groups);
    l.spp = (l.nseg + l.parts - 1) / l.parts;
    l.parts = (l.nseg + l.spp - 1) / l.spp;  // no empty part
    // kBlsSub sub-parts of up to sspp segments tile each part (the last ones may be short or empty)
    l.sspp = l.parts > 1 ? (l.spp + kBlsSub - 1) / kBlsSub : l.spp;
    l.subs = l.parts > 1 ? l.parts * kBlsSub : 1;
    int64_t o = 0;
    l.off_bc = 0;  // no widened copy of B / C
    l.off_ck = o;
    if (!given_ck) o = bwd_align(o + s.batch * s.dim * l.nseg * s.dstate * 4);
    l.off_bcpart = o;
    o = bwd_align(o + l.groups * s.batch * 2 * s.dstate * l.lp * 4);
    l.off_apart = o;
    o = bwd_align(o + l.parts * s.batch * s.dim * s.dstate * 4);
    l.off_dpart = o;
    o = bwd_align(o + l.parts * s.batch * s.dim * 4);
    l.off_bpart = o;
    o = bwd_align(o + l.parts * s.batch * s.dim * 4);
    l.off_carry = o;
    if (l.subs > 1) o = bwd_align(o + 2 * (l.subs - 1) * s.batch * s.dim * s.dstate * 4);
    l.total = o;
    return l;
}

}  // namespace mscan
