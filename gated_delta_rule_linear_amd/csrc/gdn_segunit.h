// Which unit one workgroup of a pass over the backward's units takes: head h
// of sequence n (tokens [tb, te)) or, with a time split, its segment j of P
// (tokens [sb, se)), slot the segment's slot.  Shared by the backward's sweeps
// and by the forward kernel's checkpoint pass, so both walk the same units.
#pragma once

#include "gdn_device.h"

namespace gdn {

struct SegUnit {
    int n, h, j, P, slot;
    int64_t tb, te, sb, se;
    bool valid;
};

// A: an argument struct with H, num_seqs, seg (0: no split; else a multiple of
// 64), cu (cu_seqlens), ord and pfx.  Without the split, workgroup b takes
// head b % H of sequence ord[b / H] (longest first), or of sequence b / H when
// ord is null.  With the split and pfx: head b % H of segment b / H - pfx[i] of
// sequence ord[i], pfx[i] <= b / H < pfx[i + 1] (the long sequences' segments
// first); without pfx, segment slot b / H (sequence n's segment j is slot
// cu[n] / seg + n + j).
template <class A>
__device__ __forceinline__ SegUnit seg_unit(const A& a, int b) {
    SegUnit u;
    const int H = a.H;
    const int64_t seg = a.seg;
    if (seg == 0) {
        const int nb = b / H;
        u.h = b - nb * H;
        u.n = a.ord ? a.ord[nb] : nb;
        u.tb = a.cu[u.n];
        u.te = a.cu[u.n + 1];
        u.j = u.slot = 0;
        u.P = 1;
        u.sb = u.tb;
        u.se = u.te;
        u.valid = true;
        return u;
    }
    const int s = b / H;
    u.h = b - s * H;
    if (a.pfx) {
        // the sequences in the order ord: the last i with pfx[i] <= s
        if (s >= a.pfx[a.num_seqs]) {
            u.valid = false;
            return u;
        }
        int lo = 0, hi = a.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.pfx[mid] <= s) lo = mid;
            else hi = mid - 1;
        }
        u.n = a.ord[lo];
        u.tb = a.cu[u.n];
        u.te = a.cu[u.n + 1];
        u.j = s - a.pfx[lo];
        u.P = max(1, (int)((u.te - u.tb + seg - 1) / seg));
        u.slot = (int)(u.tb / seg) + u.n + u.j;
        u.valid = u.j < u.P;
    } else {
        // the last sequence whose first slot is at or before s (first slots increase with n)
        int lo = 0, hi = a.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)a.cu[mid] / seg + mid <= s) lo = mid;
            else hi = mid - 1;
        }
        u.n = lo;
        u.tb = a.cu[lo];
        u.te = a.cu[lo + 1];
        u.j = s - (int)(u.tb / seg + lo);
        u.P = max(1, (int)((u.te - u.tb + seg - 1) / seg));
        u.slot = s;
        u.valid = u.j >= 0 && u.j < u.P;
    }
    u.sb = u.tb + (int64_t)u.j * seg;
    u.se = u.sb + seg < u.te ? u.sb + seg : u.te;
    return u;
}

}  // namespace gdn
