// ja_tiles.h -- which column range a tile of rows can see (host and device).
//
// Visibility (local indices; the library's reading of the post's masks):
// query i sees key j iff j < Lk, causal => j <= i, and window W > 0 =>
// (causal ? i - j < W : |i - j| < W).
//
// A "row tile" is [r0, min(Lr, r0 + bm)). Not transposed: rows are queries and
// columns keys (forward, dQ pass). Transposed: rows are keys and columns queries
// (the key-stationary dK/dV pass). The visible columns of a row tile always form
// one contiguous range [lo, hi), possibly empty.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define JA_HD __host__ __device__ __forceinline__
#else
#define JA_HD inline
#endif

namespace ja {

struct ColRange {
    int64_t lo, hi;  // empty when hi <= lo
};

JA_HD int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
JA_HD int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }

JA_HD ColRange visible_cols(int64_t Lr, int64_t Lc, int64_t r0, int32_t bm, int causal,
                            int32_t window, int transposed) {
    const int64_t r1 = imin64(Lr, r0 + bm);
    ColRange c{0, Lc};
    if (!transposed) {
        if (causal) c.hi = imin64(c.hi, r1);
        if (window > 0) {
            c.lo = imax64(c.lo, r0 - window + 1);
            if (!causal) c.hi = imin64(c.hi, r1 - 1 + window);
        }
    } else {
        if (causal) c.lo = imax64(c.lo, r0);
        if (window > 0) {
            c.hi = imin64(c.hi, r1 - 1 + window);
            if (!causal) c.lo = imax64(c.lo, r0 - window + 1);
        }
    }
    return c;
}

// Column tiles of width bn touched by the range: [lo/bn, ceil(hi/bn)).
JA_HD int32_t tile_cost(ColRange c, int32_t bn) {
    if (c.hi <= c.lo) return 0;
    return (int32_t)((c.hi + bn - 1) / bn - c.lo / bn);
}

// Does the (rows x cols) block [r0, r0+nr) x [c0, c0+nc) (queries x keys) contain a
// pair that is not visible, apart from rows past the sequence end (never written)?
JA_HD bool block_needs_mask(int64_t r0, int64_t nr, int64_t c0, int64_t nc, int64_t Lk,
                            int causal, int32_t window) {
    const int64_t rmax = r0 + nr - 1, cmax = c0 + nc - 1;
    if (cmax >= Lk) return true;
    if (causal && cmax > r0) return true;
    if (window > 0) {
        if (rmax - c0 >= window) return true;
        if (!causal && cmax - r0 >= window) return true;
    }
    return false;
}

// Is every pair of the block invisible?
JA_HD bool block_all_masked(int64_t r0, int64_t nr, int64_t c0, int64_t nc, int64_t Lk,
                            int causal, int32_t window) {
    const int64_t rmax = r0 + nr - 1, cmax = c0 + nc - 1;
    if (c0 >= Lk) return true;
    if (causal && c0 > rmax) return true;
    if (window > 0) {
        if (r0 - cmax >= window) return true;                 // keys all too far behind
        if (!causal && c0 - rmax >= window) return true;      // keys all too far ahead
    }
    return false;
}

}  // namespace ja
