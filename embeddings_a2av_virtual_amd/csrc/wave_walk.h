// wave_walk.h — the piece walk of the a2av copy for more than 8 ranks, one
// wave per piece of the flat destination space (destination 0's rows, then
// destination 1's, ...), written once for two kinds of wave:
//   - the GPU's 64-lane wavefront (k_a2av_wave_any in a2av.hip), and
//   - a host model of one: 64 threads in lockstep (tests/wave_walk_host.cpp),
//     which runs this very code over host buffers, checks that every
//     cross-lane operation is reached by all 64 lanes at the same place, and
//     records every copy it makes.
//
// The wave type Wv provides, per lane:
//   lane()                 this lane's index, 0..63
//   load_uniform(p)        a load of *p at an address every lane holds the same
//   copy(dst, src, n)      a copy of n bytes that all 64 lanes make together
// and operations each called by all 64 lanes at one place (site names the
// place, for the host model's check):
//   ballot(site, b)        the 64-bit mask of lanes with b set
//   readlane(site, v, l)   lane l's v
//   uniform(site, x)       x of the first lane (every lane holds the same x)
//   incl_scan(site, v)     the inclusive prefix sum of v over lanes 0..lane
//   dest_totals(site, a)   lane d < W: recv_off[d][W] (the rows destination d
//                          receives); other lanes 0
//   row(site, a, d, ro, n) lane s < W: ro = recv_off[d][s] and
//                          n = recv_off[d][s + 1] - ro; other lanes 0 (d is
//                          the same in every lane)
// How a wave comes by the offsets is its own affair: the GPU's wave takes the
// totals, and the row of the destination its workgroup starts in, from what
// the workgroup loaded once through the scalar cache; the host model loads
// them lane by lane.
//
// The argument block A provides W, R (row bytes), piece (bytes per piece),
// in[], out[], in_rows[], cap[] (per rank) and the device matrices
// recv_off ([W][W+1]) and send_off ([W][W+1]), already checked against S by
// the launch before (so recv_off[d][s+1] - recv_off[d][s] is S[s][d]).
//
// Per piece, a wave finds the destination d whose rows hold the piece's first
// byte (lanes 0..W-1 hold the rows of destinations before them), then takes
// row d of recv_off, lane s holding the first output row of source s's chunk
// and its row count; the chunk's send offset is one uniform load when the
// wave copies from it.
#pragma once

#include <stdint.h>

#include "bounds.h"

namespace a2av {

template <class Wv, class A>
A2AV_HD inline void walk_pieces_any(Wv &wv, const A &a, uint64_t gw, uint64_t TW) {
    const int lane = wv.lane();
    const int W = a.W, W1 = W + 1;
    const uint64_t R = a.R;
    const uint64_t piece = a.piece;
    // lane d: rows destination d receives, and (scanned) the rows before it
    const uint64_t tot = wv.dest_totals(11, a);
    const uint64_t incl = wv.incl_scan(1, tot);
    const uint64_t pre = incl - tot;
    const uint64_t B = wv.readlane(2, incl, 63) * R;
    for (uint64_t p = gw; p * piece < B; p += TW) {
        const uint64_t lo = p * piece;
        const uint64_t hi = lo + piece < B ? lo + piece : B;
        // last destination starting at or before lo (lane 0 always qualifies
        // once the offsets are valid)
        const uint64_t mask_d = wv.ballot(3, lane < W && pre * R <= lo);
        if (mask_d == 0) break;
        int d = 63 - __builtin_clzll(mask_d);
        uint64_t dbase = wv.readlane(4, pre, d) * R;
        // lane s: first output row of source s's chunk in destination d, and
        // its rows
        uint64_t ro, n;
        wv.row(12, a, d, ro, n);
        // last source chunk starting at or before lo
        const uint64_t mask_s = wv.ballot(5, lane < W && dbase + ro * R <= lo);
        if (mask_s == 0) break;
        int s = 63 - __builtin_clzll(mask_s);
        uint64_t x = lo;
        while (x < hi && d < W) {
            const uint64_t nn = wv.readlane(6, n, s);
            const uint64_t r0 = wv.readlane(7, ro, s);
            const uint64_t F = dbase + r0 * R;
            const uint64_t L = nn * R;
            if (nn > 0 && x < F + L) {
                const uint64_t e = hi < F + L ? hi : F + L;
                const uint64_t off = x - F;
                // d and s are the same in every lane: saying so keeps the
                // argument reads and the offset load below uniform
                const int du = wv.uniform(8, d);
                const int su = wv.uniform(9, s);
                const uint64_t s0 = (uint64_t)wv.load_uniform(a.send_off + (uint64_t)su * W1 + du);
                // checked offsets always pass; this keeps every access inside
                // the caller's buffers regardless (the offsets are re-read
                // from the caller's memory), with no sum that can wrap; both
                // sides are evaluated (no short cut), so their loads go out
                // together
                const bool fits = span_fits(r0, nn, (uint64_t)a.cap[du]) &
                                  span_fits(s0, nn, (uint64_t)a.in_rows[su]);
                if (fits) wv.copy(a.out[du] + r0 * R + off, a.in[su] + s0 * R + off, e - x);
                x = e;
            }
            if (++s == W) {
                s = 0;
                if (++d < W && x < hi) {
                    dbase = wv.readlane(10, pre, d) * R;
                    wv.row(13, a, d, ro, n);
                }
            }
        }
    }
}

}  // namespace a2av
