// ja_common.h -- device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core conventions (CDNA3/CDNA4 32x32 MFMA, wave64):
//   A operand (32 rows x K): lane l supplies row l%32; lane group g = l/32 supplies
//     KPACK consecutive k slots.
//   B operand (K x 32 cols): lane l supplies column l%32, the same k slots.
//   C/D (32x32 fp32, 16 registers): lane l holds column l%32, register r holds
//     row 8*(r/4) + 4*g + r%4.
// The kernels only rely on A and B pairing the same (group, slot) with the same k,
// so the k-order inside one instruction never matters to them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Race-check build switch: with JA_SINGLE_STAGE=1 the forward and both backward
// passes stream every stage (K/V, or Q/dO) through one LDS buffer, loaded and then
// consumed between two workgroup barriers, instead of double buffering (the next
// stage loading while the current one is consumed). The arithmetic is the same, so
// the two builds must agree bit for bit; a missing wait or barrier in the
// double-buffered path would show as a difference.
#ifndef JA_SINGLE_STAGE
#define JA_SINGLE_STAGE 0
#endif

namespace ja {

constexpr bool kSingleStage = JA_SINGLE_STAGE != 0;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One 32x32xK matrix-core step for element type T.
template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int KPACK = 8;  // elements per lane per operand
    typedef bf16x8 frag;
    static __device__ __forceinline__ floatx16 run(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int KPACK = 1;
    typedef float frag;
    static __device__ __forceinline__ floatx16 run(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// Row of the C tile held by register r of a lane in group g.
__device__ __forceinline__ constexpr int c_row(int g, int r) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Key permutation inside a 32-key block. The score tile S^T = K Q^T puts keys on
// C rows; loading A-row rho with key kappa(rho) makes register r of group g hold key
// 2*KPACK*(r/KPACK) + KPACK*g + r%KPACK, so that a lane's KPACK keys for one P*V
// step are contiguous (one vector LDS read of V^T).
template <int KPACK>
__device__ __forceinline__ constexpr int key_of_reg(int g, int r) {
    return 2 * KPACK * (r / KPACK) + KPACK * g + (r % KPACK);
}

template <int KPACK>
__device__ __forceinline__ constexpr int key_of_arow(int rho) {
    return key_of_reg<KPACK>((rho >> 2) & 1, 4 * (rho >> 3) + (rho & 3));
}

// Reductions across the two halves of a wave (lanes l and l^32 hold the same
// column of a C tile).
__device__ __forceinline__ float xhalf_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float xhalf_sum(float x) { return x + __shfl_xor(x, 32); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Pointwise activations in the GDPA form: x * sigmoid(z), with z = x for SiLU and
// z = 2 sqrt(2/pi) (x + 0.044715 x^3) for tanh-GELU (0.5 (1 + tanh u) = sigmoid(2u)).
// ACT_GELU_TAYLOR is the ALU-only GELU of the same section: the Taylor
// polynomial of the tanh form about 0 through x^6, x/2 + k2 x^2 + k4 x^4 + k6 x^6
// with c = sqrt(2/pi), a = 0.044715: k2 = c/2, k4 = (c a - c^3/3)/2,
// k6 = (2 c^5/15 - c^3 a)/2. No transcendental instruction; meant for inputs
// that QK-norm keeps small (within 1.2e-3 of the tanh form for |x| <= 1).
enum { ACT_SOFTMAX = 0, ACT_SILU = 1, ACT_GELU = 2, ACT_GELU_TAYLOR = 3 };

constexpr float kGeluK2 = 0.398942280401432678f;
constexpr float kGeluK4 = -0.0668194771775045642f;
constexpr float kGeluK6 = 0.0102015571062664970f;

template <int ACT>
__device__ __forceinline__ float pointwise(float x) {
    if (ACT == ACT_GELU_TAYLOR) {
        const float t = x * x;
        const float u = fmaf(fmaf(kGeluK6, t, kGeluK4), t, kGeluK2);
        return fmaf(t, u, 0.5f * x);
    }
    float z;
    if (ACT == ACT_SILU) {
        z = x;
    } else {
        const float c2 = 1.5957691216057308f;  // 2 * sqrt(2/pi)
        z = c2 * fmaf(0.044715f * x, x * x, x);
    }
    return x * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

// Activation and its derivative for the backward. Both activations have the form
// act(x) = x s(w(x)) with s the logistic function: w = x for SiLU, and for the
// tanh GELU w = 2 sqrt(2/pi) (x + 0.044715 x^3), because (1 + tanh(u)) / 2 =
// s(2u). Then act'(x) = s (1 + x (1 - s) w'(x)). For large |x| s saturates to
// exactly 0 or 1 and both results stay finite.
template <int ACT>
__device__ __forceinline__ void pointwise_grad(float x, float& a, float& da) {
    if (ACT == ACT_GELU_TAYLOR) {
        const float t = x * x;
        a = fmaf(t, fmaf(fmaf(kGeluK6, t, kGeluK4), t, kGeluK2), 0.5f * x);
        da = fmaf(x, fmaf(fmaf(6.0f * kGeluK6, t, 4.0f * kGeluK4), t, 2.0f * kGeluK2), 0.5f);
        return;
    }
    float w, dw;
    if (ACT == ACT_SILU) {
        w = x;
        dw = 1.0f;
    } else {
        const float c2 = 1.5957691216057308f;  // 2 * sqrt(2/pi)
        const float x2 = x * x;
        w = c2 * fmaf(0.044715f * x, x2, x);
        dw = c2 * fmaf(3.0f * 0.044715f, x2, 1.0f);
    }
    const float sg = fast_rcp(1.0f + fast_exp2(-w * kLog2e));
    a = x * sg;
    da = sg * fmaf(x * (1.0f - sg), dw, 1.0f);
}

// Block-uniform scalar broadcast helpers.
__device__ __forceinline__ int readfirstlane(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace ja
