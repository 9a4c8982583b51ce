// ja_tiles.h -- which column range a tile of rows can see (host and device).
//
// Visibility (local indices; the library's reading of the post's masks):
// query i sees key j iff j < Lk, causal => j <= i, window W > 0 =>
// (causal ? i - j < W : |i - j| < W), and with blocks of 2^bsh tokens
// ("BlockAttention": each query block attends only to its own key/value block)
// (i >> bsh) == (j >> bsh). bsh = kNoBlock disables the block mask.
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

constexpr int kNoBlock = 31;  // block shift that puts every index below 2^31 in block 0

JA_HD int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
JA_HD int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }

JA_HD ColRange visible_cols(int64_t Lr, int64_t Lc, int64_t r0, int32_t bm, int causal,
                            int32_t window, int transposed, int bsh = kNoBlock) {
    const int64_t r1 = imin64(Lr, r0 + bm);
    ColRange c{0, Lc};
    if (bsh < kNoBlock && r1 > r0) {  // columns of the blocks the rows lie in
        c.lo = imax64(c.lo, (r0 >> bsh) << bsh);
        c.hi = imin64(c.hi, (((r1 - 1) >> bsh) + 1) << bsh);
    }
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

// The visibility rule taken for one fixed query row or one fixed key: what it
// sees is always one contiguous index range, so testing an element costs one
// subtract and one unsigned compare. The kernels compute these once per work
// item; bsh is the block shift (kNoBlock: no block mask).
struct VisRange {
    int lo, width;  // x visible iff lo <= x < lo + width (width >= 0, lo >= 0)
    JA_HD bool has(int x) const { return (uint32_t)(x - lo) < (uint32_t)width; }
    // Does the range miss every index of [x0, x0 + n) / contain all of them (n > 0)?
    JA_HD bool misses(int x0, int n) const { return width == 0 || x0 >= lo + width || x0 + n <= lo; }
    JA_HD bool covers(int x0, int n) const { return x0 >= lo && x0 + n <= lo + width; }
};

JA_HD VisRange make_range(int64_t lo, int64_t hi) {
    lo = lo < 0 ? 0 : lo;
    return VisRange{(int)lo, (int)(hi > lo ? hi - lo : 0)};
}

// Keys (of Lk) that query `row` sees.
JA_HD VisRange keys_seen_by(int row, int Lk, int causal, int window, int bsh) {
    int64_t lo = 0, hi = Lk;
    if (causal) hi = hi < (int64_t)row + 1 ? hi : (int64_t)row + 1;
    if (window > 0) {
        lo = (int64_t)row - window + 1;
        if (!causal) hi = hi < (int64_t)row + window ? hi : (int64_t)row + window;
    }
    if (bsh < kNoBlock) {
        const int64_t b0 = (int64_t)(row >> bsh) << bsh, b1 = b0 + ((int64_t)1 << bsh);
        lo = lo > b0 ? lo : b0;
        hi = hi < b1 ? hi : b1;
    }
    return make_range(lo, hi);
}

// Queries (of Lq) that see `key` (none when key >= Lk).
JA_HD VisRange queries_seeing(int key, int Lq, int Lk, int causal, int window, int bsh) {
    int64_t lo = 0, hi = key < Lk ? Lq : 0;
    if (causal) lo = key;
    if (window > 0) {
        hi = hi < (int64_t)key + window ? hi : (int64_t)key + window;
        if (!causal) lo = (int64_t)key - window + 1;
    }
    if (bsh < kNoBlock) {
        const int64_t b0 = (int64_t)(key >> bsh) << bsh, b1 = b0 + ((int64_t)1 << bsh);
        lo = lo > b0 ? lo : b0;
        hi = hi < b1 ? hi : b1;
    }
    return make_range(lo, hi);
}

}  // namespace ja
