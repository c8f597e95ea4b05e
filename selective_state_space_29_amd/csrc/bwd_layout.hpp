// Workspace layout of the backward pass (host side), shared by its launcher and the C-ABI entry
// points that size and check the caller's workspace.
#pragma once

#include <stdint.h>

#include "../../include/mamba_scan.h"

namespace mscan {

constexpr int kBwdSeg = 16;  // steps per segment (checkpoint interval)

struct BwdLayout {
    int64_t lp, nseg, groups;
    int64_t off_bc, off_ck, off_bcpart, off_apart, off_dpart, off_bpart, total;
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

}  // namespace mscan
