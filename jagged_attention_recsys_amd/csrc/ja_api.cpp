// ja_api.cpp -- the C ABI declared in include/jagged_attn.h.
//
// Host side only: argument validation (everything checkable without reading
// device memory), workspace layout, kernel selection and launches. No call
// allocates, frees or synchronises, except ja_validate_offsets, which is
// synchronous by contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <vector>

#include "jagged_attn.h"
#include "ja_block.h"
#include "ja_internal.h"
#include "ja_mx.h"
#include "ja_tiles.h"

using namespace ja;

namespace {

constexpr size_t kWsAlign = 256;

// Events recorded around the attention kernels (ja_set_profile_events).
thread_local hipEvent_t g_prof_before = nullptr;
thread_local hipEvent_t g_prof_mid = nullptr;
thread_local hipEvent_t g_prof_after = nullptr;
constexpr int kMaxDevices = 64;

size_t align_up(size_t x) { return (x + kWsAlign - 1) & ~(kWsAlign - 1); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct FwdPlan {
    int layout;  // kLayoutStandard / kLayoutSplit / kLayoutChunked
    FwdShape shape;
    int64_t max_pairs;
    size_t off_tbase, off_items, bytes;
};

// Forward layout from the sizes alone (never from device data): short-query batches
// (mean query length <= 48, e.g. pooled attention seeds) use the split layout;
// short keys and values with long queries (mean key length <= 64, one stage, and
// mean query length >= 512, e.g. cross-attention to a few events) use the chunked
// layout. Every layout is correct for any lengths; the choice only affects speed.
int fwd_layout(int32_t B, int64_t Tq, int64_t Tk, int32_t dtype) {
    if (dtype != JA_BF16 || B <= 0) return kLayoutStandard;
    if (Tq <= 48LL * B) return kLayoutSplit;
    if (Tk <= 64LL * B && Tq >= 512LL * B) return kLayoutChunked;
    return kLayoutStandard;
}

// Token rows of at most 2^20 elements (H d): the kernels form 32-bit byte offsets of
// up to 256 rows (4 bytes per element) inside a stage.
constexpr int64_t kMaxRowElems = 1 << 20;

ja_status_t check_common(int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk, int32_t act,
                         int32_t window, float scale, int32_t dtype) {
    if (B < 0 || H < 1 || Tq < 0 || Tk < 0 || window < 0) return JA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return JA_ERR_INVALID_ARG;
    if (Tq > INT32_MAX || Tk > INT32_MAX || (int64_t)H * d > kMaxRowElems) return JA_ERR_UNSUPPORTED;
    if (!fwd_supported(dtype, d, act)) return JA_ERR_UNSUPPORTED;
    return JA_OK;
}

ja_status_t plan_fwd(int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk, int32_t act, int32_t dtype,
                     FwdPlan* p) {
    p->layout = fwd_layout(B, Tq, Tk, dtype);
    p->shape = fwd_shape(dtype, d, act, p->layout);
    if (p->shape.bm <= 0) return JA_ERR_UNSUPPORTED;
    p->max_pairs = (Tq + p->shape.bm - 1) / p->shape.bm + B;
    if (p->max_pairs * (int64_t)H >= INT32_MAX) return JA_ERR_UNSUPPORTED;
    p->off_tbase = align_up(sizeof(int32_t) * kCtrCount);
    p->off_items = align_up(p->off_tbase + sizeof(int32_t) * ((size_t)B + 1));
    p->bytes = align_up(p->off_items + sizeof(int32_t) * kItemInts * (size_t)p->max_pairs);
    return JA_OK;
}

struct BwdPlan {
    int rows, cols;                     // rows per item, columns per stage
    int64_t max_q_pairs, max_k_pairs;
    size_t off_qctr, off_kctr, off_qtbase, off_ktbase, off_qitems, off_kitems, off_di, off_nl2, bytes;
};

ja_status_t plan_bwd(int32_t B, int32_t H, int64_t Tq, int64_t Tk, BwdPlan* p) {
    p->rows = bwd_rows_per_item();
    p->cols = bwd_cols_per_stage();
    p->max_q_pairs = (Tq + p->rows - 1) / p->rows + B;
    p->max_k_pairs = (Tk + p->rows - 1) / p->rows + B;
    if (p->max_q_pairs * (int64_t)H >= INT32_MAX || p->max_k_pairs * (int64_t)H >= INT32_MAX)
        return JA_ERR_UNSUPPORTED;
    size_t o = 0;
    p->off_qctr = o; o = align_up(o + sizeof(int32_t) * kCtrCount);
    p->off_kctr = o; o = align_up(o + sizeof(int32_t) * kCtrCount);
    p->off_qtbase = o; o = align_up(o + sizeof(int32_t) * ((size_t)B + 1));
    p->off_ktbase = o; o = align_up(o + sizeof(int32_t) * ((size_t)B + 1));
    p->off_qitems = o; o = align_up(o + sizeof(int32_t) * kItemInts * (size_t)p->max_q_pairs);
    p->off_kitems = o; o = align_up(o + sizeof(int32_t) * kItemInts * (size_t)p->max_k_pairs);
    p->off_di = o; o = align_up(o + sizeof(float) * (size_t)Tq * (size_t)H);
    p->off_nl2 = o; o = align_up(o + sizeof(float) * (size_t)Tq * (size_t)H);
    p->bytes = o;
    return JA_OK;
}

struct BlkPlan {
    int64_t max_pairs;  // (sequence, 64-token tile) pairs at most
    size_t off_tbase, off_items, bytes;
};

ja_status_t plan_blk(int32_t B, int32_t H, int64_t T, BlkPlan* p) {
    p->max_pairs = (T + kBlkTile - 1) / kBlkTile + B;
    if (p->max_pairs * (int64_t)H >= INT32_MAX) return JA_ERR_UNSUPPORTED;
    p->off_tbase = align_up(sizeof(int32_t) * kCtrCount);
    p->off_items = align_up(p->off_tbase + sizeof(int32_t) * ((size_t)B + 1));
    p->bytes = align_up(p->off_items + sizeof(int32_t) * kItemInts * (size_t)p->max_pairs);
    return JA_OK;
}

int device_cus() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int fwd_occupancy(int dtype, int d, int act, int layout) {
    static std::atomic<int> cache[2][3][4][3];
    const int di = d == 32 ? 0 : d == 64 ? 1 : 2;
    std::atomic<int>& slot = cache[dtype][di][act][layout];
    int n = slot.load(std::memory_order_relaxed);
    if (n > 0) return n;
    n = fwd_blocks_per_cu(dtype, d, act, layout);
    slot.store(n, std::memory_order_relaxed);
    return n;
}

int blk_occupancy_cached(int d) {
    static std::atomic<int> cache[3];
    std::atomic<int>& slot = cache[d == 32 ? 0 : d == 64 ? 1 : 2];
    int n = slot.load(std::memory_order_relaxed);
    if (n > 0) return n;
    n = blk_blocks_per_cu(d);
    slot.store(n, std::memory_order_relaxed);
    return n;
}

SchedArgs sched_args(const FwdPlan& p, const int32_t* q_offsets, const int32_t* k_offsets, int32_t B,
                     int32_t H, int32_t causal, int32_t window, int32_t bsh, void* workspace) {
    char* ws = static_cast<char*>(workspace);
    SchedArgs s;
    s.row_off = q_offsets;
    s.col_off = k_offsets;
    s.B = B;
    s.H = H;
    s.bm = p.shape.bm;
    s.bn = p.shape.bn;
    s.causal = causal ? 1 : 0;
    s.window = window;
    s.transposed = 0;
    s.bsh = bsh;
    s.max_pairs = p.max_pairs;
    s.tbase = reinterpret_cast<int32_t*>(ws + p.off_tbase);
    s.items = reinterpret_cast<int32_t*>(ws + p.off_items);
    s.counters = reinterpret_cast<int32_t*>(ws);
    return s;
}

// log2 of a block size that is a power of two in [1, 2^30], else -1.
int block_shift(int32_t block) {
    if (block < 1 || (block & (block - 1)) != 0) return -1;
    int sh = 0;
    while ((1 << sh) < block) ++sh;
    return sh;
}

}  // namespace

namespace ja {

// Every check of the forward's arguments that needs no device access, workspace
// aside; JA_OK also for an empty batch (the caller then has nothing to do).
ja_status_t fwd_check_args(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                           const int32_t* k_offsets, int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                           int32_t act, int32_t window, float scale, int32_t dtype, const void* out, const float* lse) {
    ja_status_t st = check_common(B, H, d, Tq, Tk, act, window, scale, dtype);
    if (st != JA_OK) return st;
    if (B == 0 || Tq == 0) return JA_OK;  // no query rows: nothing to write
    if (!q || !out || !q_offsets || !k_offsets) return JA_ERR_INVALID_ARG;
    if (Tk > 0 && (!k || !v)) return JA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
        !aligned(q_offsets, 4) || !aligned(k_offsets, 4))
        return JA_ERR_INVALID_ARG;
    return JA_OK;
}

}  // namespace ja

namespace {

ja_status_t fwd_impl(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                     const int32_t* k_offsets, int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                     int32_t act, int32_t causal, int32_t window, int32_t bsh, float scale, int32_t dtype, void* out,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    ja_status_t st = fwd_check_args(q, k, v, q_offsets, k_offsets, B, H, d, Tq, Tk, act, window, scale, dtype, out,
                                    lse);
    if (st != JA_OK) return st;
    if (B == 0 || Tq == 0) return JA_OK;  // no query rows: nothing to write
    if (!workspace || !aligned(workspace, 16)) return JA_ERR_INVALID_ARG;
    FwdPlan p;
    st = plan_fwd(B, H, d, Tq, Tk, act, dtype, &p);
    if (st != JA_OK) return st;
    if (workspace_bytes < p.bytes) return JA_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    SchedArgs sa = sched_args(p, q_offsets, k_offsets, B, H, causal, window, bsh, workspace);
    if (launch_sched(sa, s) != hipSuccess) return JA_ERR_HIP;

    FwdArgs fa;
    fa.q = q;
    fa.k = k;
    fa.v = v;
    fa.out = out;
    fa.lse = act == JA_ACT_SOFTMAX ? lse : nullptr;
    fa.q_off = q_offsets;
    fa.k_off = k_offsets;
    fa.items = sa.items;
    fa.counters = sa.counters;
    fa.H = H;
    fa.Tq = (int32_t)Tq;
    fa.Tk = (int32_t)Tk;
    fa.causal = causal ? 1 : 0;
    fa.window = window;
    fa.bsh = bsh;
    fa.scale = scale;
    const int64_t max_items = p.max_pairs * H;
    int64_t grid = (int64_t)device_cus() * fwd_occupancy(dtype, d, act, p.layout);
    if (grid > max_items) grid = max_items;
    if (grid < 1) grid = 1;
    if (g_prof_before && hipEventRecord(g_prof_before, s) != hipSuccess) return JA_ERR_HIP;
    if (launch_fwd(fa, dtype, d, act, p.layout, (int)grid, s) != hipSuccess) return JA_ERR_HIP;
    if (g_prof_after && hipEventRecord(g_prof_after, s) != hipSuccess) return JA_ERR_HIP;
    return JA_OK;
}

ja_status_t bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, const int32_t* q_offsets, const int32_t* k_offsets, int32_t B, int32_t H,
                     int32_t d, int64_t Tq, int64_t Tk, int32_t act, int32_t causal, int32_t window, int32_t bsh,
                     float scale, int32_t dtype, int32_t grad_dtype, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, void* stream) {
    ja_status_t st = check_common(B, H, d, Tq, Tk, act, window, scale, dtype);
    if (st != JA_OK) return st;
    if (!bwd_supported(dtype, d, act)) return JA_ERR_UNSUPPORTED;
    if (grad_dtype != dtype && grad_dtype != JA_F32) return JA_ERR_UNSUPPORTED;
    if (B == 0 || (Tq == 0 && Tk == 0)) return JA_OK;
    if (!q_offsets || !k_offsets || !workspace) return JA_ERR_INVALID_ARG;
    const bool softmax = act == JA_ACT_SOFTMAX;  // only softmax reads the forward's out and lse
    if (Tq > 0 && (!q || !dout || !dq || (softmax && (!out || !lse)))) return JA_ERR_INVALID_ARG;
    if (Tk > 0 && (!k || !v || !dk || !dv)) return JA_ERR_INVALID_ARG;
    const void* ptrs16[] = {q, k, v, softmax ? out : nullptr, dout, dq, dk, dv, workspace};
    for (const void* p16 : ptrs16)
        if (!aligned(p16, 16)) return JA_ERR_INVALID_ARG;
    if ((softmax && !aligned(lse, 4)) || !aligned(q_offsets, 4) || !aligned(k_offsets, 4))
        return JA_ERR_INVALID_ARG;
    BwdPlan p;
    st = plan_bwd(B, H, Tq, Tk, &p);
    if (st != JA_OK) return st;
    if (workspace_bytes < p.bytes) return JA_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    SchedArgs sq;
    sq.row_off = q_offsets;
    sq.col_off = k_offsets;
    sq.B = B;
    sq.H = H;
    sq.bm = p.rows;
    sq.bn = p.cols;
    sq.causal = causal ? 1 : 0;
    sq.window = window;
    sq.transposed = 0;
    sq.bsh = bsh;
    sq.max_pairs = p.max_q_pairs;
    sq.tbase = reinterpret_cast<int32_t*>(ws + p.off_qtbase);
    sq.items = reinterpret_cast<int32_t*>(ws + p.off_qitems);
    sq.counters = reinterpret_cast<int32_t*>(ws + p.off_qctr);
    SchedArgs sk = sq;
    sk.row_off = k_offsets;
    sk.col_off = q_offsets;
    sk.transposed = 1;
    sk.max_pairs = p.max_k_pairs;
    sk.tbase = reinterpret_cast<int32_t*>(ws + p.off_ktbase);
    sk.items = reinterpret_cast<int32_t*>(ws + p.off_kitems);
    sk.counters = reinterpret_cast<int32_t*>(ws + p.off_kctr);
    if (launch_sched2(sq, sk, s) != hipSuccess) return JA_ERR_HIP;

    BwdArgs ba;
    ba.q = q;
    ba.k = k;
    ba.v = v;
    ba.out = softmax ? out : nullptr;
    ba.dout = dout;
    ba.lse = softmax ? lse : nullptr;
    ba.dq = dq;
    ba.dk = dk;
    ba.dv = dv;
    ba.di = reinterpret_cast<float*>(ws + p.off_di);
    ba.nl2 = reinterpret_cast<float*>(ws + p.off_nl2);
    ba.q_off = q_offsets;
    ba.k_off = k_offsets;
    ba.q_items = sq.items;
    ba.k_items = sk.items;
    ba.q_counters = sq.counters;
    ba.k_counters = sk.counters;
    ba.H = H;
    ba.Tq = (int32_t)Tq;
    ba.Tk = (int32_t)Tk;
    ba.causal = causal ? 1 : 0;
    ba.window = window;
    ba.bsh = bsh;
    ba.scale = scale;
    ba.grad_f32 = grad_dtype == JA_F32 ? 1 : 0;
    // d = 128 with keys longer than one stage on average: the role-split dK/dV pass
    // (two waves per SIMD). Short key tiles keep the four-wave pass, whose wave
    // pairs split the query stages of tiles of at most 64 keys.
    ba.kv_roles = (d == 128 && Tk > 64LL * B) ? 1 : 0;
    const int64_t cap_q = (int64_t)device_cus() * bwd_blocks_per_cu(d, act, false, ba.grad_f32 != 0, false);
    const int64_t cap_k =
        (int64_t)device_cus() * bwd_blocks_per_cu(d, act, true, ba.grad_f32 != 0, ba.kv_roles != 0);
    int64_t gq = p.max_q_pairs * H, gk = p.max_k_pairs * H;
    gq = gq < cap_q ? gq : cap_q;
    gk = gk < cap_k ? gk : cap_k;
    if (gq < 1) gq = 1;
    if (gk < 1) gk = 1;
    if (launch_bwd(ba, d, act, (int)gq, (int)gk, s, g_prof_before, g_prof_mid, g_prof_after) != hipSuccess)
        return JA_ERR_HIP;
    return JA_OK;
}

// Block-diagonal attention with blocks of at most kBlkTile tokens: the tile
// scheduler lists the 64-token tiles, then one workgroup per (tile, head).
ja_status_t blk_schedule(const int32_t* offsets, int32_t B, int32_t H, int64_t T, int32_t causal, int32_t bsh,
                         void* workspace, size_t workspace_bytes, hipStream_t s, BlkArgs* ba, int64_t* grid) {
    BlkPlan p;
    ja_status_t st = plan_blk(B, H, T, &p);
    if (st != JA_OK) return st;
    if (workspace_bytes < p.bytes) return JA_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    SchedArgs sa;
    sa.row_off = offsets;
    sa.col_off = offsets;
    sa.B = B;
    sa.H = H;
    sa.bm = kBlkTile;
    sa.bn = kBlkTile;
    sa.causal = causal ? 1 : 0;
    sa.window = 0;
    sa.transposed = 0;
    sa.bsh = bsh;
    sa.max_pairs = p.max_pairs;
    sa.tbase = reinterpret_cast<int32_t*>(ws + p.off_tbase);
    sa.items = reinterpret_cast<int32_t*>(ws + p.off_items);
    sa.counters = reinterpret_cast<int32_t*>(ws);
    if (launch_sched(sa, s) != hipSuccess) return JA_ERR_HIP;
    *ba = BlkArgs{};
    ba->off = offsets;
    ba->items = sa.items;
    ba->counters = sa.counters;
    ba->B = B;
    ba->H = H;
    ba->T = (int32_t)T;
    ba->causal = causal ? 1 : 0;
    ba->bsh = bsh;
    ba->cap = (int32_t)(p.max_pairs * H);
    *grid = p.max_pairs * H;
    return JA_OK;
}

}  // namespace

extern "C" {

size_t ja_fwd_workspace_size(int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk, int32_t act,
                             int32_t causal, int32_t window, int32_t dtype) {
    (void)causal;
    if (check_common(B, H, d, Tq, Tk, act, window, 1.0f, dtype) != JA_OK) return 0;
    FwdPlan p;
    if (plan_fwd(B, H, d, Tq, Tk, act, dtype, &p) != JA_OK) return 0;
    return p.bytes;
}

ja_status_t jagged_attn_fwd(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                            const int32_t* k_offsets, int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                            int32_t act, int32_t causal, int32_t window, float scale, int32_t dtype, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_impl(q, k, v, q_offsets, k_offsets, B, H, d, Tq, Tk, act, causal, window, kNoBlock, scale, dtype,
                    out, lse, workspace, workspace_bytes, stream);
}

ja_status_t jagged_block_attn_fwd(const void* q, const void* k, const void* v, const int32_t* offsets, int32_t B,
                                  int32_t H, int32_t d, int64_t T, int32_t block, int32_t causal, float scale,
                                  int32_t dtype, void* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    const int bsh = block_shift(block);
    if (bsh < 0) return JA_ERR_INVALID_ARG;
    return fwd_impl(q, k, v, offsets, offsets, B, H, d, T, T, JA_ACT_SOFTMAX, causal, 0, bsh, scale, dtype, out,
                    lse, workspace, workspace_bytes, stream);
}

size_t ja_block_attn_workspace_size(int32_t B, int32_t H, int32_t d, int64_t T, int32_t block, int32_t causal,
                                    int32_t dtype) {
    (void)causal;
    if (block_shift(block) < 0) return 0;
    if (check_common(B, H, d, T, T, JA_ACT_SOFTMAX, 0, 1.0f, dtype) != JA_OK) return 0;
    size_t bytes = 0;
    FwdPlan fp;
    if (plan_fwd(B, H, d, T, T, JA_ACT_SOFTMAX, dtype, &fp) != JA_OK) return 0;
    bytes = fp.bytes;
    if (bwd_supported(dtype, d, JA_ACT_SOFTMAX)) {
        BwdPlan bp;
        if (plan_bwd(B, H, T, T, &bp) != JA_OK) return 0;
        bytes = bp.bytes > bytes ? bp.bytes : bytes;
    }
    BlkPlan kp;
    if (plan_blk(B, H, T, &kp) != JA_OK) return 0;
    return kp.bytes > bytes ? kp.bytes : bytes;
}

size_t ja_bwd_workspace_size(int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk, int32_t act,
                             int32_t causal, int32_t window, int32_t dtype) {
    (void)causal;
    if (check_common(B, H, d, Tq, Tk, act, window, 1.0f, dtype) != JA_OK) return 0;
    if (!bwd_supported(dtype, d, act)) return 0;
    BwdPlan p;
    if (plan_bwd(B, H, Tq, Tk, &p) != JA_OK) return 0;
    return p.bytes;
}

ja_status_t jagged_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                            const float* lse, const int32_t* q_offsets, const int32_t* k_offsets, int32_t B,
                            int32_t H, int32_t d, int64_t Tq, int64_t Tk, int32_t act, int32_t causal,
                            int32_t window, float scale, int32_t dtype, int32_t grad_dtype, void* dq, void* dk,
                            void* dv, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_impl(q, k, v, out, dout, lse, q_offsets, k_offsets, B, H, d, Tq, Tk, act, causal, window, kNoBlock,
                    scale, dtype, grad_dtype, dq, dk, dv, workspace, workspace_bytes, stream);
}

ja_status_t jagged_block_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                  const float* lse, const int32_t* offsets, int32_t B, int32_t H, int32_t d,
                                  int64_t T, int32_t block, int32_t causal, float scale, int32_t dtype, void* dq,
                                  void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
    const int bsh = block_shift(block);
    if (bsh < 0) return JA_ERR_INVALID_ARG;
    if (!blk_supported(dtype, d, bsh))
        return bwd_impl(q, k, v, out, dout, lse, offsets, offsets, B, H, d, T, T, JA_ACT_SOFTMAX, causal, 0, bsh,
                        scale, dtype, dtype, dq, dk, dv, workspace, workspace_bytes, stream);
    ja_status_t st = check_common(B, H, d, T, T, JA_ACT_SOFTMAX, 0, scale, dtype);
    if (st != JA_OK) return st;
    if (B == 0 || T == 0) return JA_OK;
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !offsets || !workspace) return JA_ERR_INVALID_ARG;
    const void* ptrs16[] = {q, k, v, dout, dq, dk, dv, workspace};
    for (const void* p16 : ptrs16)
        if (!aligned(p16, 16)) return JA_ERR_INVALID_ARG;
    if (!aligned(offsets, 4)) return JA_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    BlkArgs ba;
    int64_t grid = 0;
    st = blk_schedule(offsets, B, H, T, causal, bsh, workspace, workspace_bytes, s, &ba, &grid);
    if (st != JA_OK) return st;
    ba.q = q;
    ba.k = k;
    ba.v = v;
    ba.dout = dout;
    ba.dq = dq;
    ba.dk = dk;
    ba.dv = dv;
    ba.scale = scale;
    if (g_prof_before && hipEventRecord(g_prof_before, s) != hipSuccess) return JA_ERR_HIP;
    const int64_t cap_bwd = (int64_t)device_cus() * blk_occupancy_cached(d);
    if (grid > cap_bwd) grid = cap_bwd;
    if (launch_blk_bwd(ba, d, (int)grid, s) != hipSuccess) return JA_ERR_HIP;
    if (g_prof_after && hipEventRecord(g_prof_after, s) != hipSuccess) return JA_ERR_HIP;
    return JA_OK;
}

size_t ja_mxfp8_quantize_workspace_size(int32_t B, int64_t T) {
    if (B < 0 || T < 0) return 0;
    const int64_t blocks = (T + kMxBlock - 1) / kMxBlock + B;
    if (blocks >= INT32_MAX) return 0;
    return align_up(sizeof(int32_t) * (size_t)(blocks > 0 ? blocks : 1));
}

ja_status_t ja_mxfp8_quantize(const void* x, int32_t dtype, const int32_t* offsets, int32_t B, int32_t H, int32_t d,
                              int64_t T, void* x8, void* scales, int32_t* scale_offsets, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (B < 0 || H < 1 || T < 0 || d < kMxBlock || d % kMxBlock != 0) return JA_ERR_INVALID_ARG;
    if ((int64_t)H * d > kMaxRowElems) return JA_ERR_UNSUPPORTED;
    if (dtype != JA_BF16) return JA_ERR_UNSUPPORTED;
    if (T > INT32_MAX) return JA_ERR_UNSUPPORTED;
    if (!offsets || !scale_offsets || (T > 0 && (!x || !x8 || !scales)) || !workspace) return JA_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(offsets, 4) || !aligned(scale_offsets, 4) ||
        !aligned(workspace, 4))
        return JA_ERR_INVALID_ARG;
    const int64_t blocks = (T + kMxBlock - 1) / kMxBlock + B;
    if (blocks >= INT32_MAX || blocks * H * (d / kMxBlock) >= INT32_MAX) return JA_ERR_UNSUPPORTED;
    if (workspace_bytes < sizeof(int32_t) * (size_t)(blocks > 0 ? blocks : 1)) return JA_ERR_WORKSPACE;
    MxQuantArgs a;
    a.x = x;
    a.off = offsets;
    a.x8 = static_cast<uint8_t*>(x8);
    a.scales = static_cast<uint8_t*>(scales);
    a.soff = scale_offsets;
    a.blk_seq = static_cast<int32_t*>(workspace);
    a.B = B;
    a.H = H;
    a.d = d;
    a.T = (int32_t)T;
    a.max_blocks = (int32_t)blocks;
    if (launch_mx_quant(a, static_cast<hipStream_t>(stream)) != hipSuccess) return JA_ERR_HIP;
    return JA_OK;
}

size_t ja_fwd_mxfp8_workspace_size(int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk) {
    if (B < 0 || H < 1 || d != kMxD || Tq < 0 || Tk < 0 || Tq > INT32_MAX || Tk > INT32_MAX) return 0;
    if ((int64_t)H * d > kMaxRowElems) return 0;
    const int64_t max_pairs = (Tq + kMxBM - 1) / kMxBM + B;
    if (max_pairs * (int64_t)H >= INT32_MAX) return 0;
    const size_t off_tbase = align_up(sizeof(int32_t) * kCtrCount);
    const size_t off_items = align_up(off_tbase + sizeof(int32_t) * ((size_t)B + 1));
    return align_up(off_items + sizeof(int32_t) * kItemInts * (size_t)max_pairs);
}

ja_status_t jagged_attn_fwd_mxfp8(const void* q8, const void* q_scales, const int32_t* q_scale_offsets,
                                  const void* k8, const void* k_scales, const int32_t* k_scale_offsets,
                                  const void* v8, const void* v_scales, const int32_t* q_offsets,
                                  const int32_t* k_offsets, int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                                  int32_t causal, int32_t window, float scale, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || H < 1 || Tq < 0 || Tk < 0 || window < 0 || !std::isfinite(scale)) return JA_ERR_INVALID_ARG;
    if (d != kMxD) return JA_ERR_UNSUPPORTED;
    if (Tq > INT32_MAX || Tk > INT32_MAX || (int64_t)H * d > kMaxRowElems) return JA_ERR_UNSUPPORTED;
    if (B == 0 || Tq == 0) return JA_OK;
    if (!q8 || !q_scales || !q_scale_offsets || !out || !q_offsets || !k_offsets || !k_scale_offsets || !workspace)
        return JA_ERR_INVALID_ARG;
    if (Tk > 0 && (!k8 || !v8 || !k_scales || !v_scales)) return JA_ERR_INVALID_ARG;
    const void* p16[] = {q8, k8, v8, out, workspace};
    for (const void* p : p16)
        if (!aligned(p, 16)) return JA_ERR_INVALID_ARG;
    const void* p4[] = {q_scales, k_scales, v_scales, q_scale_offsets, k_scale_offsets, q_offsets, k_offsets, lse};
    for (const void* p : p4)
        if (!aligned(p, 4)) return JA_ERR_INVALID_ARG;
    const size_t need = ja_fwd_mxfp8_workspace_size(B, H, d, Tq, Tk);
    if (need == 0) return JA_ERR_UNSUPPORTED;
    if (workspace_bytes < need) return JA_ERR_WORKSPACE;
    const int64_t max_pairs = (Tq + kMxBM - 1) / kMxBM + B;
    char* ws = static_cast<char*>(workspace);
    SchedArgs sa;
    sa.row_off = q_offsets;
    sa.col_off = k_offsets;
    sa.B = B;
    sa.H = H;
    sa.bm = kMxBM;
    sa.bn = kMxKT;
    sa.causal = causal ? 1 : 0;
    sa.window = window;
    sa.transposed = 0;
    sa.bsh = kNoBlock;
    sa.max_pairs = max_pairs;
    sa.counters = reinterpret_cast<int32_t*>(ws);
    sa.tbase = reinterpret_cast<int32_t*>(ws + align_up(sizeof(int32_t) * kCtrCount));
    sa.items = reinterpret_cast<int32_t*>(ws + align_up(align_up(sizeof(int32_t) * kCtrCount) +
                                                        sizeof(int32_t) * ((size_t)B + 1)));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_sched(sa, s) != hipSuccess) return JA_ERR_HIP;
    MxFwdArgs a;
    a.q8 = static_cast<const uint8_t*>(q8);
    a.k8 = static_cast<const uint8_t*>(k8);
    a.v8 = static_cast<const uint8_t*>(v8);
    a.qs = static_cast<const uint8_t*>(q_scales);
    a.ks = static_cast<const uint8_t*>(k_scales);
    a.vs = static_cast<const uint8_t*>(v_scales);
    a.q_soff = q_scale_offsets;
    a.k_soff = k_scale_offsets;
    a.out = out;
    a.lse = lse;
    a.q_off = q_offsets;
    a.k_off = k_offsets;
    a.items = sa.items;
    a.counters = sa.counters;
    a.H = H;
    a.Tq = (int32_t)Tq;
    a.Tk = (int32_t)Tk;
    a.causal = causal ? 1 : 0;
    a.window = window;
    a.scale = scale;
    static std::atomic<int> occ{0};
    int n = occ.load(std::memory_order_relaxed);
    if (n <= 0) {
        n = mx_fwd_blocks_per_cu();
        occ.store(n, std::memory_order_relaxed);
    }
    int64_t grid = (int64_t)device_cus() * n;
    if (grid > max_pairs * H) grid = max_pairs * H;
    if (grid < 1) grid = 1;
    if (g_prof_before && hipEventRecord(g_prof_before, s) != hipSuccess) return JA_ERR_HIP;
    if (launch_mx_fwd(a, (int)grid, s) != hipSuccess) return JA_ERR_HIP;
    if (g_prof_after && hipEventRecord(g_prof_after, s) != hipSuccess) return JA_ERR_HIP;
    return JA_OK;
}

ja_status_t ja_fwd_schedule(const int32_t* q_offsets, const int32_t* k_offsets, int32_t B, int32_t H, int32_t d,
                            int64_t Tq, int64_t Tk, int32_t act, int32_t causal, int32_t window, int32_t dtype,
                            int32_t* items, int32_t* count, int64_t max_items, void* workspace,
                            size_t workspace_bytes, void* stream) {
    ja_status_t st = check_common(B, H, d, Tq, Tk, act, window, 1.0f, dtype);
    if (st != JA_OK) return st;
    if (!q_offsets || !k_offsets || !items || !count || !workspace) return JA_ERR_INVALID_ARG;
    FwdPlan p;
    st = plan_fwd(B, H, d, Tq, Tk, act, dtype, &p);
    if (st != JA_OK) return st;
    if (max_items < p.max_pairs) return JA_ERR_INVALID_ARG;
    if (workspace_bytes < p.bytes) return JA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    SchedArgs sa = sched_args(p, q_offsets, k_offsets, B, H, causal, window, kNoBlock, workspace);
    if (launch_sched(sa, s) != hipSuccess) return JA_ERR_HIP;
    if (launch_copy_items(sa.counters, sa.items, items, count, max_items, s) != hipSuccess) return JA_ERR_HIP;
    return JA_OK;
}

ja_status_t ja_fwd_tile_shape(int32_t B, int32_t d, int64_t Tq, int64_t Tk, int32_t act, int32_t dtype,
                              int32_t* bm, int32_t* bn) {
    if (!bm || !bn || B < 0 || Tq < 0 || Tk < 0) return JA_ERR_INVALID_ARG;
    if (!fwd_supported(dtype, d, act)) return JA_ERR_UNSUPPORTED;
    FwdShape s = fwd_shape(dtype, d, act, fwd_layout(B, Tq, Tk, dtype));
    *bm = s.bm;
    *bn = s.bn;
    return JA_OK;
}

ja_status_t ja_validate_offsets(const int32_t* offsets, int32_t B, int64_t T, void* stream) {
    if (!offsets || B < 0 || T < 0) return JA_ERR_INVALID_ARG;
    std::vector<int32_t> h((size_t)B + 1);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(h.data(), offsets, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, s) != hipSuccess)
        return JA_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return JA_ERR_HIP;
    if (h[0] != 0 || (int64_t)h[B] != T) return JA_ERR_INVALID_OFFSETS;
    for (int32_t b = 0; b < B; ++b)
        if (h[b + 1] < h[b]) return JA_ERR_INVALID_OFFSETS;
    return JA_OK;
}

void ja_set_profile_events(void* before, void* after) {
    g_prof_before = static_cast<hipEvent_t>(before);
    g_prof_mid = nullptr;
    g_prof_after = static_cast<hipEvent_t>(after);
}

void ja_set_profile_events3(void* before, void* mid, void* after) {
    g_prof_before = static_cast<hipEvent_t>(before);
    g_prof_mid = static_cast<hipEvent_t>(mid);
    g_prof_after = static_cast<hipEvent_t>(after);
}

size_t ja_probe_mfma_workspace_size(void) {
    const size_t groups = (size_t)device_cus();
    return align_up(sizeof(uint64_t) * 2 * groups) + sizeof(float) * groups * (size_t)probe_threads();
}

ja_status_t ja_probe_mfma(int32_t iters, void* workspace, size_t workspace_bytes, int32_t* groups,
                          int64_t* flop_per_group, int32_t* wallclock_khz, void* stream) {
    if (iters < 1 || !workspace || !groups || !flop_per_group || !wallclock_khz || !aligned(workspace, 16))
        return JA_ERR_INVALID_ARG;
    const int g = device_cus();
    const size_t off_sink = align_up(sizeof(uint64_t) * 2 * (size_t)g);
    if (workspace_bytes < off_sink + sizeof(float) * (size_t)g * (size_t)probe_threads()) return JA_ERR_WORKSPACE;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        return JA_ERR_HIP;
    char* ws = static_cast<char*>(workspace);
    if (launch_probe_mfma(iters, g, reinterpret_cast<uint64_t*>(ws), reinterpret_cast<float*>(ws + off_sink),
                          static_cast<hipStream_t>(stream)) != hipSuccess)
        return JA_ERR_HIP;
    *groups = g;
    *flop_per_group = (int64_t)iters * probe_flop_per_iter();
    *wallclock_khz = khz;
    return JA_OK;
}

const char* ja_status_string(ja_status_t status) {
    switch (status) {
        case JA_OK: return "ok";
        case JA_ERR_INVALID_ARG: return "invalid argument";
        case JA_ERR_UNSUPPORTED: return "unsupported configuration";
        case JA_ERR_WORKSPACE: return "workspace too small";
        case JA_ERR_INVALID_OFFSETS: return "malformed offsets";
        case JA_ERR_HIP: return "HIP runtime error";
        case JA_ERR_SCRATCH: return "sizes need more workspace than the fixed no-alloc buffer holds";
    }
    return "unknown status";
}

int32_t ja_version(void) { return 100; }

}  // extern "C"
