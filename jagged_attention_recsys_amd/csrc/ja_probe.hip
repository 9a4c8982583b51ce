// ja_probe.hip -- machine figures the benchmark reports beside its results: the
// bf16 matrix-core rate a plain stream of 32x32x16 products sustains on every SIMD
// and the shader clock the GPU runs at while doing it.
//
// One workgroup of four waves per compute unit (the LDS it reserves keeps a
// second one off the unit), so every SIMD runs exactly one wave. Each wave issues
// `iters` rounds of kAcc independent accumulations (no memory traffic inside the
// loop). Wave 0 of each workgroup reads the shader cycle counter and the constant
// real-time counter before and after its loop; the host turns the two deltas into
// the clock frequency. The accumulators are written out so that the products
// cannot be removed.
#include "ja_common.h"

namespace ja {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kAcc = 4;  // independent accumulator chains per wave

__global__ __launch_bounds__(kProbeThreads) void ja_probe_mfma_kernel(int iters, uint64_t* out, float* sink) {
#if defined(__HIP_DEVICE_COMPILE__)
    __shared__ float reserve[96 * 256];  // 96 KB: one workgroup per compute unit
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (iters < 0) reserve[threadIdx.x] = 0.0f;  // never taken; keeps the reservation
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (bf16)(0.001f * (float)(lane + i));
        b[i] = (bf16)(0.002f * (float)(lane - i));
    }
    floatx16 acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = floatx16{};
    uint64_t c0 = 0, r0 = 0;
    if (wave == 0) {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    if (wave == 0) {
        // the counters are read after the loop's results exist
        asm volatile("" ::"v"(s));
        const uint64_t c1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) {
            out[2 * blockIdx.x] = c1 - c0;
            out[2 * blockIdx.x + 1] = r1 - r0;
        }
    }
    sink[blockIdx.x * kProbeThreads + threadIdx.x] = s + reserve[threadIdx.x & 1] * 0.0f;
#else
    (void)iters;
    (void)out;
    (void)sink;
#endif
}

}  // namespace

int probe_threads() { return kProbeThreads; }
int probe_flop_per_iter() { return kAcc * 32 * 32 * 16 * 2 * (kProbeThreads / 64); }

hipError_t launch_probe_mfma(int iters, int grid, uint64_t* out, float* sink, hipStream_t stream) {
    hipLaunchKernelGGL(ja_probe_mfma_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, iters, out, sink);
    return hipGetLastError();
}

}  // namespace ja
