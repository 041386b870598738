// Order in which the persistent prefill grids take their work items.
//
// A work item is one query tile of one (batch, head).  Its length is the
// number of key tiles it sweeps: under the causal mask, proportional to the
// tile's position, so items are ranked longest-first (rank t counts query
// tiles from the last one).  Workgroups are dispatched round-robin over the
// 8 XCDs of the chip (workgroup w runs on XCD w mod 8) and each XCD has its
// own L2, so where the items of a head run decides how often its K and V
// are fetched from HBM.
//
// Head-major (when the head count and the grid are multiples of 8): head bh
// belongs to XCD bh mod 8.  The S = G/8 workgroups of an XCD take that XCD's
// items head by head, longest first, in a snake: in round r, slot s takes
// item r S + s (even r) or r S + S - 1 - s (odd r).  All slots of an XCD
// start sweeping the keys of one head together and advance at about the same
// rate, so each K and V tile comes from HBM into that L2 about once per
// round and serves the other slots from there; and over a pair of rounds a
// slot's long item is paired with a short one, which evens out the causal
// lengths.
//
// Otherwise: one snake over all items sorted longest-first (round r takes
// items r G .. r G + G - 1, reversed on odd rounds within each XCD), so every
// workgroup still gets an even share of the causal work.
#pragma once

namespace diffattn {

// Item of workgroup w (of G) in round r: sets t (longest-first rank of the
// query tile) and bh; returns false when the workgroup has no more items.
__device__ __forceinline__ bool prefill_item(int r, int w, int G, int nqt, int BH, int& t, int& bh) {
    if ((G & 7) == 0 && (BH & 7) == 0) {
        const int S = G >> 3, xcd = w & 7, slot = w >> 3;
        const int i = r * S + ((r & 1) ? S - 1 - slot : slot);
        if (i >= (BH >> 3) * nqt) return false;
        const int hl = i / nqt;
        t = i - hl * nqt;
        bh = 8 * hl + xcd;
        return true;
    }
    const int w_odd = (G & 7) == 0 ? (w & 7) + 8 * (G / 8 - 1 - w / 8) : G - 1 - w;
    const int k = r * G + ((r & 1) ? w_odd : w);
    if (k >= nqt * BH) return false;
    t = k / BH;
    bh = k - t * BH;
    return true;
}

}  // namespace diffattn
