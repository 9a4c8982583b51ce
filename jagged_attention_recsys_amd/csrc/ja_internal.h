// ja_internal.h -- interfaces between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "jagged_attn.h"

namespace ja {

// Scheduler cost bins: costs at or above kSchedBins-1 share the last bin.
constexpr int kSchedBins = 512;

// Slots of the counter block at the start of every workspace.
// Work-list counters: total items, the single pop counter, list length, and eight
// per-XCD pop counters (64 bytes apart) for kernels that pop from XCD-local queues.
enum { kCtrTotal = 0, kCtrPop = 1, kCtrPairs = 2, kCtrQueue = 16, kCtrQueueStride = 16, kXcds = 8,
       kCtrCount = kCtrQueue + kXcds * kCtrQueueStride };

// One work item of a scheduled list: {sequence b, tile t, row_off[b], row_off[b+1],
// col_off[b], col_off[b+1], 0, 0}. Carrying the sequence's offsets lets a kernel
// read everything it needs about an item in one 32-byte load.
constexpr int kItemInts = 8;

struct SchedArgs {
    const int32_t* row_off;  // [B+1] offsets of the tiled dimension
    const int32_t* col_off;  // [B+1] offsets of the visited dimension
    int32_t B, H;
    int32_t bm, bn;          // row tile, column tile (cost unit)
    int32_t causal, window, transposed;
    int32_t bsh;             // block shift of the block-diagonal mask (kNoBlock: none)
    int64_t max_pairs;       // capacity of items; a larger enumeration schedules nothing
    int32_t* tbase;          // [B+1] scratch: first flat tile of each sequence
    int32_t* items;          // [kItemInts * max_pairs] item records
    int32_t* counters;       // kCtrCount ints
};

hipError_t launch_sched(const SchedArgs& a, hipStream_t stream);
// Both lists in one launch (one workgroup each; the lists must not share memory).
hipError_t launch_sched2(const SchedArgs& a, const SchedArgs& b, hipStream_t stream);
hipError_t launch_copy_items(const int32_t* counters, const int32_t* items, int32_t* out,
                             int32_t* count, int64_t max_items, hipStream_t stream);

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;                // may be null
    const int32_t* q_off;
    const int32_t* k_off;
    const int32_t* items;      // (sequence, q-tile) pairs
    int32_t* counters;
    int32_t H;
    int32_t Tq, Tk;            // tensor extents: rows outside [0, T) are never touched
    int32_t causal, window;
    int32_t bsh;               // block shift of the block-diagonal mask (kNoBlock: none)
    float scale;               // applied to Q K^T
};

// Forward kernel family. `layout` selects the standard layout (0: four 32-row query
// slices sharing each key tile), the short-query layout (1: one 32-row query tile
// per workgroup, the waves splitting the keys) or the short-key layout (2: items of
// several consecutive query tiles sharing one resident key/value stage).
enum { kLayoutStandard = 0, kLayoutSplit = 1, kLayoutChunked = 2 };
struct FwdShape {
    int bm;  // query rows per work item
    int bn;  // keys per stage (scheduler cost unit)
};
bool fwd_supported(int dtype, int d, int act);
FwdShape fwd_shape(int dtype, int d, int act, int layout);
hipError_t launch_fwd(const FwdArgs& a, int dtype, int d, int act, int layout, int grid,
                      hipStream_t stream);
// Workgroups per CU the forward kernel reaches (from the occupancy query).
int fwd_blocks_per_cu(int dtype, int d, int act, int layout);

// Softmax backward: dQ pass (query tiles) then dK/dV pass (key tiles).
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;          // forward log-sum-exp, natural log, [Tq, H]
    void* dq;
    void* dk;
    void* dv;
    float* di;                 // workspace [Tq, H]: rowsum(dO * O), written by the dQ pass
    float* nl2;                // workspace [Tq, H]: -lse * log2(e), written by the dQ pass (softmax)
    const int32_t* q_off;
    const int32_t* k_off;
    const int32_t* q_items;    // (sequence, query tile) pairs
    const int32_t* k_items;    // (sequence, key tile) pairs
    int32_t* q_counters;
    int32_t* k_counters;
    int32_t H;
    int32_t Tq, Tk;
    int32_t causal, window;
    int32_t bsh;               // block shift of the block-diagonal mask (kNoBlock: none)
    float scale;
    int32_t grad_f32;          // dq, dk, dv are fp32 (else the input type)
    int32_t kv_roles;          // d = 128: the dK/dV pass in its role-split form (8 waves, 2 per SIMD)
};
bool bwd_supported(int dtype, int d, int act);
int bwd_rows_per_item();   // query rows (dQ pass) and key rows (dK/dV pass) per work item
int bwd_cols_per_stage();  // keys (dQ pass) and queries (dK/dV pass) per stage: scheduler cost unit
// Events (may be null) recorded before the dQ pass, between the passes and after
// the dK/dV pass.
hipError_t launch_bwd(const BwdArgs& a, int d, int act, int grid_q, int grid_k, hipStream_t stream,
                      hipEvent_t before, hipEvent_t mid, hipEvent_t after);
// Workgroups per CU of the dQ (false) or dK/dV pass (roles: its role-split form).
int bwd_blocks_per_cu(int d, int act, bool dkdv, bool grad_f32, bool roles);

// Argument checks of jagged_attn_fwd that need no device access (workspace aside);
// JA_OK also for an empty batch.
ja_status_t fwd_check_args(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                           const int32_t* k_offsets, int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                           int32_t act, int32_t window, float scale, int32_t dtype, const void* out, const float* lse);

// Machine probe: one workgroup per compute unit streaming 32x32x16 bf16 products;
// writes (shader cycles, real-time ticks) of each workgroup's loop to out[2 g],
// out[2 g + 1]; sink receives probe_threads() floats per workgroup.
int probe_threads();
int probe_flop_per_iter();  // matrix flop one workgroup performs per iteration
hipError_t launch_probe_mfma(int iters, int grid, uint64_t* out, float* sink, hipStream_t stream);

}  // namespace ja
