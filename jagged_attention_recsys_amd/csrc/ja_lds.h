// ja_lds.h -- LDS tiles of token rows and the matrix-operand reads on them.
//
// A tile holds ROWS consecutive token rows of one head (K, V, Q or dO), d
// contiguous, streamed from HBM by buffer loads straight into LDS. Each row's
// 16-byte chunks are XOR-swizzled (swz) so that the two read patterns the
// kernels use are free of bank conflicts:
//   * row-operand reads (A operand "rows x d" of a 32x32x16 product): lane l
//     reads 8 bf16 of row kappa(l%32) at d-chunk 2s + l/32;
//   * transpose reads (A operand "d x rows"): ds_read_tr16_b64, each 16-lane
//     group gathering 4 rows x 16 dims, twice for 8 rows.
// Rows past the end of the sequence read as zero: the buffer descriptor of a
// tile ends at the sequence's last row.
#pragma once

#include "ja_common.h"
#include "ja_internal.h"
#include "ja_tiles.h"

namespace ja {

typedef __attribute__((address_space(3))) char lds_char;
typedef short shortx4 __attribute__((ext_vector_type(4)));

template <typename T> struct Frag;
template <> struct Frag<bf16> {
    typedef bf16x8 type;
    static __device__ __forceinline__ type zero() { return type{}; }
};
template <> struct Frag<float> {
    typedef float type;
    static __device__ __forceinline__ type zero() { return 0.0f; }
};

// XOR swizzle of the 16-byte chunks of an LDS row (bf16 rows of 4, 8 or 16
// chunks; fp32 tiles are not swizzled). The LDS serves 64 banks of 4 bytes per
// cycle: 16 lanes of a 16-byte read, or 32 lanes of an 8-byte read. The swizzle
// keeps both read patterns free of bank conflicts:
//   * row-operand reads (16 lanes): 16 rows at one fixed chunk land on 16
//     distinct 16-byte bank groups;
//   * transpose reads (32 lanes): 4 consecutive rows (4-aligned) x 4 consecutive
//     chunks (4-aligned) land on 16 distinct groups.
template <int CPR, int ESZ>
__device__ __forceinline__ int swz(int row) {
    if (ESZ != 2) return 0;
    if (CPR == 16) return ((row & 3) << 2) | ((row >> 2) & 3);        // 256-B rows
    if (CPR == 8) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);  // 128-B rows, 2 per bank cycle
    return (row >> 2) & 3;                                            // 64-B rows, 4 per bank cycle
}

template <typename T, int D, int ROWS>
struct Tile {
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int KP = Mma<T>::KPACK;
    static constexpr int ROWB = D * ESZ;           // bytes per row
    static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
    static constexpr int BYTES = ROWS * ROWB;
    static constexpr int INSTR = BYTES / 1024;     // 64-lane x 16-byte loads per tile
    static constexpr int NS = D / (2 * KP);        // k-steps over d
    static constexpr int ND = D / 32;              // 32-row blocks over d
    static_assert(BYTES % 1024 == 0, "tile must be whole 64-lane loads");

    // Row-operand offsets of lane (col, grp) inside a 32-row block, per k-step.
    static __device__ __forceinline__ void row_offsets(int col, int grp, int (&off)[NS]) {
        const int r = key_of_arow<KP>(col);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if constexpr (KP == 8) {
                const int c = 2 * s + grp;
                off[s] = r * ROWB + ((c ^ swz<CPR, ESZ>(r)) << 4);
            } else {
                off[s] = r * ROWB + (2 * s + grp) * 4;
            }
        }
    }

    // Row-operand offsets in one register (bf16, 256-byte rows): the lane's offset
    // for k-step s is rx ^ (s << 5). The swizzle only permutes chunk bits 5-7 of the
    // row, which the row base leaves clear, so the XOR form equals row_offsets.
    static __device__ __forceinline__ int row_offset_base(int col, int grp) {
        static_assert(KP == 8 && CPR == 16, "bf16 rows of 256 bytes");
        const int r = key_of_arow<KP>(col);
        return r * ROWB + ((grp ^ swz<CPR, ESZ>(r)) << 4);
    }
    static __device__ __forceinline__ int row_offset(int rx, int s) { return rx ^ (s << 5); }

    // Transpose-read offsets (bf16) of lane l inside a 16-row step, per 32-dim
    // block and row quad; fp32 tiles read single elements instead.
    static __device__ __forceinline__ void tr_offsets(int lane, int (&off)[ND][2]) {
        const int grp = lane >> 5, col = lane & 31;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {
                if constexpr (KP == 8) {
                    const int i = lane & 15, cb = (lane >> 4) & 1;
                    const int row = 8 * grp + 4 * hq + (i >> 2);
                    const int d = 32 * db + 16 * cb + 4 * (i & 3);
                    off[db][hq] = row * ROWB + (((d >> 3) ^ swz<CPR, ESZ>(row)) << 4) + 8 * ((d >> 2) & 1);
                } else {
                    off[db][hq] = grp * ROWB + (32 * db + col) * 4;
                }
            }
    }

    // A operand "rows x d" of k-step s for the 32-row block starting at blk.
    static __device__ __forceinline__ typename Frag<T>::type read_rows(const char* blk, int off) {
        return *(const typename Frag<T>::type*)(blk + off);
    }

    // A operand "d x rows" for k-step t over the 32-row block at blk (rows
    // 16t + 8grp + 0..7 in the key_of_reg order), 32-dim block db.
    static __device__ __forceinline__ typename Frag<T>::type read_tr(const char* blk, int t, const int (&off)[ND][2],
                                                                    int db) {
        if constexpr (KP == 8) {
            const char* base = blk + 16 * t * ROWB;
            const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) shortx4*)(base + off[db][0]));
            const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) shortx4*)(base + off[db][1]));
            return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0, 1,
                                           2, 3, 4, 5, 6, 7);
        } else {
            return *(const float*)(blk + 2 * t * ROWB + off[db][0]);
        }
    }
};

// Per-lane global byte offsets of the chunks this lane loads for a tile, for
// each of its (at most LPW) 64-lane loads; load j of wave w is tile load
// w + j*NW.
template <typename TileT, int NW>
struct TileLoader {
    static constexpr int LPW = (TileT::INSTR + NW - 1) / NW;
    uint32_t voff[LPW];

    __device__ __forceinline__ void init(int wave, int lane, uint32_t row_stride_bytes) {
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int slot = (wave + j * NW) * 64 + lane;
            const int row = slot / TileT::CPR, p = slot % TileT::CPR;
            voff[j] = (uint32_t)row * row_stride_bytes +
                      (uint32_t)((p ^ swz<TileT::CPR, TileT::ESZ>(row)) << 4);
        }
    }

    // Rows [0, nvalid) of the tile start at `src` (row stride fixed at init);
    // rows at or past nvalid read as zero.
    __device__ __forceinline__ void issue(const char* src, uint32_t nrec_bytes, char* dst, int wave) const {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, (int)nrec_bytes, 0x00020000);
        lds_char* d = (lds_char*)dst;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int inst = wave + j * NW;
            if (TileT::INSTR % NW == 0 || inst < TileT::INSTR)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d + inst * 1024, 16, voff[j], 0, 0, 0);
        }
    }
};

// A work item's sequence, from its record (read with one 32-byte load): for a list
// tiled over queries the record's row offsets are the query offsets; for a list
// tiled over keys (transposed) they are the key offsets. Rows are clamped to the
// tensors, so inconsistent offsets cannot reach outside them (the C ABI leaves
// such offsets undefined otherwise).
struct ItemSeq {
    int b, t;        // sequence, tile
    int64_t qo, ko;  // first query / key row of the sequence
    int Lq, Lk;      // its query / key counts
};

template <typename R>
__device__ __forceinline__ ItemSeq item_from_record(const R& it, bool transposed, int Tq, int Tk) {
    const int q0 = transposed ? it[4] : it[2], q1 = transposed ? it[5] : it[3];
    const int k0 = transposed ? it[2] : it[4], k1 = transposed ? it[3] : it[5];
    ItemSeq s;
    s.b = it[0];
    s.t = it[1];
    s.qo = q0;
    s.ko = k0;
    s.Lq = q0 < 0 ? 0 : min(q1, Tq) - q0;
    s.Lk = k0 < 0 ? 0 : min(k1, Tk) - k0;
    return s;
}

__device__ __forceinline__ ItemSeq load_item(const int32_t* items, int pair, bool transposed, int Tq, int Tk) {
    typedef int int8v __attribute__((ext_vector_type(8)));
    const int8v it = *(const int8v*)(items + kItemInts * (int64_t)pair);
    return item_from_record(it, transposed, Tq, Tk);
}

// Work queues over a longest-first list of `total` items, either one for the whole grid
// or XCD-local: for XCD-local queues, queue q holds the
// items 8k + q in order, so each queue is itself longest-first and the queues are
// balanced. A workgroup pops from the queue of the XCD it runs on, and once that queue
// is empty from another queue that still holds items; every item is handed out
// exactly once. All tiles of one (sequence, head) at H = 8 (every other tile at H = 4)
// then run on one XCD, whose L2 keeps the K / V stages they share. Thread 0 of a
// workgroup does the popping: the queue it pops from and whether all queues are empty
// live in two ints of LDS (`st`), and only the pending pop's return value is held in a
// register, so a pop can be sent well before its result is needed.
__device__ __forceinline__ int xcd_id() {
    int x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return x & (kXcds - 1);
}
// local = false: one queue for the whole grid (the list's own counter).
__device__ __forceinline__ void xq_init(int* st, bool local) {
    st[0] = local ? xcd_id() : -1;  // current queue (-1: the single queue)
    st[1] = 0;                      // set once every queue was found empty
}
// Sends a pop to the current queue; the returned value goes to xq_resolve.
__device__ __forceinline__ int xq_issue(int32_t* counters, const int* st) {
    const int q = st[0];
    return atomicAdd(q < 0 ? &counters[kCtrPop] : &counters[kCtrQueue + q * kCtrQueueStride], 1);
}
// The popped item, or total once every queue is empty. When the current queue runs dry,
// the other queues' counters are read together (one round trip, not one per queue) and
// the first that still holds items is popped; a workgroup that finds them all empty is
// done.
__device__ __forceinline__ int xq_resolve(int32_t* counters, int* st, int pend, int total) {
    const int cur = st[0];
    if (cur < 0) return pend < total ? pend : total;
    if ((int64_t)kXcds * pend + cur < total) return kXcds * pend + cur;
    if (st[1]) return total;  // every queue was found empty before
    int32_t* ctr = counters + kCtrQueue;
    int seen[kXcds];
#pragma unroll
    for (int q = 0; q < kXcds; ++q) seen[q] = atomicAdd(&ctr[q * kCtrQueueStride], 0);
#pragma unroll
    for (int i = 1; i < kXcds; ++i) {
        const int q = (cur + i) & (kXcds - 1);
        const int len = (total - q + kXcds - 1) / kXcds;  // items 8k + q below total
        if (seen[q] < len) {
            const int k = atomicAdd(&ctr[q * kCtrQueueStride], 1);
            if (k < len) {
                st[0] = q;
                return kXcds * k + q;
            }
        }
    }
    st[1] = 1;
    return total;
}

// Wave-uniform mask decisions for a block [x0, x0 + n) of the other index, from
// every lane's visible range; lanes with lane_ok false (rows past the sequence
// end, never written) take no part.
__device__ __forceinline__ bool wave_skips(const VisRange& v, bool lane_ok, int x0, int n) {
    return __all(!lane_ok || v.misses(x0, n));
}
__device__ __forceinline__ bool wave_needs_mask(const VisRange& v, bool lane_ok, int x0, int n) {
    return __any(lane_ok && !v.covers(x0, n));
}

// Reductions over lanes l and l^32 (the two halves of a C-tile column).
__device__ __forceinline__ float halves_max(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <typename T> __device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16>(bf16* dst, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (bf16)a;
    v[1] = (bf16)b;
    v[2] = (bf16)c;
    v[3] = (bf16)d;
    *(bf16x4*)dst = v;
}
template <> __device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
    floatx4 v;
    v[0] = a;
    v[1] = b;
    v[2] = c;
    v[3] = d;
    *(floatx4*)dst = v;
}

// Convert 8 consecutive fp32 C-registers (r0..r0+7) to a bf16 B-operand fragment
// (fp32: the single register r0).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type to_frag(const floatx16& c, int r0) {
    if constexpr (Mma<T>::KPACK == 8) {
        typename Frag<T>::type f;
#pragma unroll
        for (int s = 0; s < 8; ++s) f[s] = (bf16)c[r0 + s];
        return f;
    } else {
        return c[r0];
    }
}

// A lane value the compiler cannot move out of the enclosing loop. The swizzled
// LDS addresses of the row turnarounds below depend on it, so they are computed
// where they are used instead of being held in registers through a stage loop.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Whole-row turnaround of a wave's 32 rows of one head through a wave-private LDS
// region of 32 x ROWB bytes. Global memory sees only whole rows, 16 bytes per lane
// (CPR lanes per row), instead of the 8- or 16-byte pieces of 32 rows that the
// matrix-core layouts (lane = row) would give one instruction. 16-byte chunks are
// XOR-swizzled by row: at d = 128 the 16-byte row pieces and per-lane fragments hit
// distinct banks (a model of the 64-bank LDS), while the 8-byte accumulator writes
// can pair rows r and r + 16 on one bank (a layout that separates them measured the
// same LDS bank-conflict count and time).
template <int D>
struct RowTurn {
    static constexpr int ROWB = D * 2;       // bf16 row
    static constexpr int CPR = ROWB / 16;    // 16-byte chunks per row
    static constexpr int N = CPR / 2;        // pieces per lane for 32 rows
    static constexpr int BYTES = 32 * ROWB;  // region size
    static __device__ __forceinline__ int at(int r, int c) { return r * ROWB + ((c ^ (r & (CPR - 1))) << 4); }

    // Rows [0, 32) from base (row 0, this head), row stride rs elements; rows at
    // or past nrows read as zero.
    static __device__ __forceinline__ void load(bf16x8 (&raw)[N], const bf16* base, int64_t rs, int nrows,
                                                int lane) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int p = n * 64 + lane, r = p / CPR, c = p % CPR;
            raw[n] = r < nrows ? *(const bf16x8*)(base + r * rs + c * 8) : bf16x8{};
        }
    }
    static __device__ __forceinline__ void put(char* reg, const bf16x8 (&raw)[N], int lane) {
        const int ln = opaque(lane);
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int p = n * 64 + ln;
            *(bf16x8*)(reg + at(p / CPR, p % CPR)) = raw[n];
        }
    }
    // B-operand fragments: fragment s of lane (col, grp) holds elements
    // [8 grp + 16 s, 8 grp + 16 s + 8) of row col.
    static __device__ __forceinline__ void frags(bf16x8 (&f)[D / 16], const char* reg, int lane) {
        const int ln = opaque(lane), cl = ln & 31, gp = ln >> 5;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) f[s] = *(const bf16x8*)(reg + at(cl, gp + 2 * s));
    }
    // C-layout accumulators of O^T-like products (lane = row col, register r of
    // block i = element 32 i + 8 (r / 4) + 4 grp + r % 4), times sc, as bf16 rows.
    static __device__ __forceinline__ void put_acc(char* reg, const floatx16 (&acc)[D / 32], float sc, int lane) {
        const int ln = opaque(lane), cl = ln & 31, gp = ln >> 5;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 v;
                v[0] = (bf16)(acc[i][4 * j] * sc);
                v[1] = (bf16)(acc[i][4 * j + 1] * sc);
                v[2] = (bf16)(acc[i][4 * j + 2] * sc);
                v[3] = (bf16)(acc[i][4 * j + 3] * sc);
                *(bf16x4*)(reg + at(cl, 4 * i + j) + gp * 8) = v;
            }
    }
    // Region rows [0, nrows) to global rows at base (row 0, this head).
    static __device__ __forceinline__ void store(bf16* base, int64_t rs, int nrows, const char* reg, int lane) {
        const int ln = opaque(lane);
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int p = n * 64 + ln, r = p / CPR, c = p % CPR;
            const bf16x8 v = *(const bf16x8*)(reg + at(r, c));
            if (r < nrows) *(bf16x8*)(base + r * rs + c * 8) = v;
        }
    }
};

}  // namespace ja
