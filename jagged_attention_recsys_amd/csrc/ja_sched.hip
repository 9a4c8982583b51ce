// ja_sched.hip -- device-side tile scheduler for jagged batches.
//
// The GDPA section of the GEM training post enumerates the valid tiles of a jagged
// batch, skips empty ones and spreads them over the GPU's compute units to remove
// load skew. Here the enumeration runs on the GPU itself (no host round trip):
// one workgroup reads the offsets, counts row tiles per sequence, gives each tile a
// cost (the number of column tiles it visits) and writes the (sequence, tile) list
// in longest-first order for a persistent grid that pops items with one atomic.
//
// Order: min(cost, kBins-1) descending, then sequence, then tile ascending. It is a
// stable counting sort: wave w of the workgroup owns a contiguous slice of the
// (sequence, tile) enumeration, so bins are laid out as (bin descending, wave
// ascending) and each wave places its items in enumeration order.
#include "ja_common.h"
#include "ja_internal.h"
#include "ja_tiles.h"

namespace ja {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
// Batches of up to kLdsSeqs sequences keep the per-sequence tile prefix and the
// offsets in LDS, so the per-tile binary search and length lookups do not wait
// on global memory; larger batches read them from the workspace and the inputs.
constexpr int kLdsSeqs = 2048;
// Enumerations of up to kLdsItems tiles (with the tables in LDS) keep each tile's
// sequence and bin from the histogram pass for the scatter pass.
constexpr int kLdsItems = 8192;

// Inclusive scan of one int per thread over the whole workgroup. `tmp` holds
// kWaves+1 ints of LDS. Returns the inclusive prefix; *total gets the sum.
__device__ int block_scan(int x, int* tmp, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int v = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    if (lane == 63) tmp[w] = v;
    __syncthreads();
    if (w == 0) {
        int t = lane < kWaves ? tmp[lane] : 0;
#pragma unroll
        for (int o = 1; o < kWaves; o <<= 1) {
            int y = __shfl_up(t, o);
            if (lane >= o) t += y;
        }
        if (lane < kWaves) tmp[lane] = t;  // inclusive wave totals
    }
    __syncthreads();
    int before = w > 0 ? tmp[w - 1] : 0;
    *total = tmp[kWaves - 1];
    __syncthreads();  // tmp may be reused right after
    return before + v;
}

// Sequence b owning flat tile f: the last b with tbase[b] <= f (tbase[B] = F > f).
__device__ int find_seq(const int32_t* tbase, int B, int f) {
    int lo = 0, hi = B;  // invariant: tbase[lo] <= f < tbase[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (tbase[mid] <= f) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Two lists (the backward's query-tile and key-tile lists) are built by one launch,
// one workgroup each; a single list uses one workgroup.
struct SchedPair {
    SchedArgs l[2];
};

__global__ __launch_bounds__(kThreads) void ja_sched_kernel(SchedPair lists) {
    const SchedArgs& a = lists.l[blockIdx.x];
    __shared__ int cnt[kWaves * kSchedBins];  // [wave][bin] counts, then offsets
    __shared__ int16_t s_seq[kLdsItems];      // per tile: its sequence and bin (cached lists)
    __shared__ int16_t s_bin[kLdsItems];
    __shared__ int tmp[kWaves + 1];
    __shared__ int32_t s_tbase[kLdsSeqs + 1];
    __shared__ int32_t s_row[kLdsSeqs + 1];
    __shared__ int32_t s_col[kLdsSeqs + 1];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool in_lds = a.B <= kLdsSeqs;

    // Phase 0: row tiles per sequence and their exclusive prefix (tbase[0..B]).
    int carry = 0;
    for (int c0 = 0; c0 <= a.B; c0 += kThreads) {
        const int b = c0 + tid;
        int n = 0;
        if (b < a.B) {
            const int64_t L = (int64_t)a.row_off[b + 1] - a.row_off[b];
            n = L > 0 ? (int)((L + a.bm - 1) / a.bm) : 0;
        }
        int total;
        int incl = block_scan(n, tmp, &total);
        if (b <= a.B) {
            a.tbase[b] = carry + incl - n;
            if (in_lds) {
                s_tbase[b] = carry + incl - n;
                s_row[b] = a.row_off[b];
                s_col[b] = a.col_off[b];
            }
        }
        carry += total;
    }
    const int32_t* tb = in_lds ? s_tbase : a.tbase;
    const int32_t* ro = in_lds ? s_row : a.row_off;
    const int32_t* co = in_lds ? s_col : a.col_off;
    // An enumeration larger than the item buffer (offsets inconsistent with the
    // sizes the host was given) schedules nothing rather than writing past it.
    const int F = (int64_t)carry <= a.max_pairs ? carry : 0;
    const bool cached = in_lds && F <= kLdsItems;
    // Column tiles are a power of two wide in every list the library builds: costs then
    // take shifts, not 64-bit divisions (the general form stays for any other width).
    const bool pow2 = (a.bn & (a.bn - 1)) == 0;
    const int lbn = pow2 ? __builtin_ctz(a.bn) : 0;
    for (int i = tid; i < kWaves * kSchedBins; i += kThreads) cnt[i] = 0;
    __threadfence_block();
    __syncthreads();

    // Each wave owns the enumeration slice [f_lo, f_hi).
    const int f_lo = (int)(((int64_t)F * w) / kWaves);
    const int f_hi = (int)(((int64_t)F * (w + 1)) / kWaves);

    auto bin_of = [&](int f, int* pb, int* pt) {
        const int b = find_seq(tb, a.B, f);
        const int t = f - tb[b];
        const int64_t Lr = (int64_t)ro[b + 1] - ro[b];
        const int64_t Lc = (int64_t)co[b + 1] - co[b];
        const ColRange cr = visible_cols(Lr, Lc, (int64_t)t * a.bm, a.bm, a.causal, a.window, a.transposed, a.bsh);
        int cost;
        if (pow2)  // 0 <= lo < hi <= Lc < 2^31: the same count as tile_cost
            cost = cr.hi <= cr.lo ? 0
                                  : (int)(((uint64_t)cr.hi + a.bn - 1) >> lbn) - (int)((uint64_t)cr.lo >> lbn);
        else
            cost = tile_cost(cr, a.bn);
        *pb = b;
        *pt = t;
        return cost < kSchedBins - 1 ? cost : kSchedBins - 1;
    };

    // Phase 1: per-wave histograms.
    for (int f = f_lo + lane; f < f_hi; f += 64) {
        int b, t;
        const int bin = bin_of(f, &b, &t);
        atomicAdd(&cnt[w * kSchedBins + bin], 1);
        if (cached) {
            s_seq[f] = (int16_t)b;
            s_bin[f] = (int16_t)bin;
        }
    }
    __syncthreads();

    // Phase 2: exclusive offsets in (bin descending, wave ascending) order. Thread
    // tid owns flat positions [8 tid, 8 tid + 8) of that order.
    {
        constexpr int per = kWaves * kSchedBins / kThreads;
        int vals[per];
        int s = 0;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            const int x = tid * per + i;
            const int bin = kSchedBins - 1 - x / kWaves, ww = x % kWaves;
            vals[i] = cnt[ww * kSchedBins + bin];
            s += vals[i];
        }
        int total;
        int incl = block_scan(s, tmp, &total);
        int run = incl - s;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            const int x = tid * per + i;
            const int bin = kSchedBins - 1 - x / kWaves, ww = x % kWaves;
            cnt[ww * kSchedBins + bin] = run;
            run += vals[i];
        }
    }
    __syncthreads();

    // Phase 3: stable scatter, one wave per slice, 64 items at a time in order.
    for (int f0 = f_lo; f0 < f_hi; f0 += 64) {
        const int f = f0 + lane;
        const bool valid = f < f_hi;
        int b = 0, t = 0, bin = -1;
        if (valid) {
            if (cached) {  // written by this lane in phase 1 (same wave, same f)
                b = s_seq[f];
                bin = s_bin[f];
                t = f - tb[b];
            } else {
                bin = bin_of(f, &b, &t);
            }
        }
        // Every lane reads its bin's next free position, learns which lanes share
        // its bin (a register-only loop over the distinct bins of the chunk), and
        // the lowest such lane advances the bin's position by their count.
        const int base = valid ? cnt[w * kSchedBins + bin] : 0;
        uint64_t pending = __ballot(valid);
        uint64_t mine = 0;
        while (pending) {
            const int leader = __ffsll((unsigned long long)pending) - 1;
            const int lbin = __builtin_amdgcn_readlane(bin, leader);
            const uint64_t same = __ballot(valid && bin == lbin);
            if (valid && bin == lbin) mine = same;
            pending &= ~same;
        }
        const uint64_t below = mine & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)));
        const int pos = base + __popcll(below);
        if (valid && below == 0) cnt[w * kSchedBins + bin] = base + __popcll(mine);
        if (valid) {
            typedef int int4v __attribute__((ext_vector_type(4)));
            int4v* rec = (int4v*)(a.items + kItemInts * (int64_t)pos);
            rec[0] = int4v{b, t, ro[b], ro[b + 1]};
            rec[1] = int4v{co[b], co[b + 1], 0, 0};
        }
    }

    if (tid == 0) {
        a.counters[kCtrTotal] = F * a.H;
        a.counters[kCtrPop] = 0;
        a.counters[kCtrPairs] = F;
    }
    if (tid < kXcds) a.counters[kCtrQueue + tid * kCtrQueueStride] = 0;
}

__global__ void ja_copy_items_kernel(const int32_t* counters, const int32_t* items, int32_t* out,
                                     int32_t* count, int64_t max_items) {
    const int F = counters[kCtrPairs];
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < F && i < max_items;
         i += (int64_t)gridDim.x * blockDim.x) {
        out[2 * i] = items[kItemInts * i];
        out[2 * i + 1] = items[kItemInts * i + 1];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *count = F;
}

}  // namespace

hipError_t launch_sched(const SchedArgs& a, hipStream_t stream) {
    SchedPair p;
    p.l[0] = a;
    p.l[1] = a;
    hipLaunchKernelGGL(ja_sched_kernel, dim3(1), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_sched2(const SchedArgs& a, const SchedArgs& b, hipStream_t stream) {
    SchedPair p;
    p.l[0] = a;
    p.l[1] = b;
    hipLaunchKernelGGL(ja_sched_kernel, dim3(2), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_copy_items(const int32_t* counters, const int32_t* items, int32_t* out,
                             int32_t* count, int64_t max_items, hipStream_t stream) {
    hipLaunchKernelGGL(ja_copy_items_kernel, dim3(64), dim3(256), 0, stream, counters, items, out,
                       count, max_items);
    return hipGetLastError();
}

}  // namespace ja
