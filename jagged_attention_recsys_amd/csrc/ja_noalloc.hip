// ja_noalloc.hip -- jagged_attn_fwd for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the forward's workspace (counters, per-sequence tile prefix, work
// list) lives in a fixed file-scope device array instead of a caller-provided
// buffer.
//
// Each GPU holds its own copy of the array, from the library's load until the
// process ends. Its device address is looked up once per device (first call made
// with that device current) and kept; host code never passes the array's own name
// to a kernel, only that looked-up address. Nothing in it needs clearing between
// calls: the tile scheduler writes every counter, prefix and work-list entry a call
// reads before the attention kernel reads it. Calls that overlap on one GPU
// (concurrent streams, several host threads) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "jagged_attn.h"
#include "ja_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)8 << 20;  // JA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == JA_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of the scratch array on the current device (nullptr on failure).
void* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

ja_status_t jagged_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                                    const int32_t* k_offsets, int32_t B, int32_t H, int32_t d, int64_t Tq,
                                    int64_t Tk, int32_t act, int32_t causal, int32_t window, float scale,
                                    int32_t dtype, void* out, float* lse, void* stream) {
    // Every host-visible check first: nothing touches the device for a call with
    // bad arguments, one that does not fit the buffer, or one with nothing to do.
    const ja_status_t st = ja::fwd_check_args(q, k, v, q_offsets, k_offsets, B, H, d, Tq, Tk, act, window, scale,
                                              dtype, out, lse);
    if (st != JA_OK) return st;
    if (B == 0 || Tq == 0) return JA_OK;
    const size_t need = ja_fwd_workspace_size(B, H, d, Tq, Tk, act, causal, window, dtype);
    if (need == 0) return JA_ERR_UNSUPPORTED;
    if (need > kScratchBytes) return JA_ERR_SCRATCH;
    void* ws = scratch_on_current_device();
    if (!ws) return JA_ERR_HIP;
    return jagged_attn_fwd(q, k, v, q_offsets, k_offsets, B, H, d, Tq, Tk, act, causal, window, scale, dtype, out,
                           lse, ws, kScratchBytes, stream);
}

}  // extern "C"
