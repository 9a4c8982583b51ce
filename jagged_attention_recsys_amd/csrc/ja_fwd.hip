// ja_fwd.hip -- fused jagged attention forward for gfx950.
//
// Computes, per (sequence, head), out = act(scale Q K^T, masks) V on the jagged
// rows of that sequence only ("Jagged Sequence Flash Attention" and "Generalized
// Dot-Product Attention (GDPA)" sections of the GEM training post): act is an
// online softmax (running max, running sum, rescaled accumulator) or a pointwise
// SiLU / tanh-GELU normalised by 1/Lk with no max, no rescale and no correction
// stage. Sliding-window and causal tiles that no query can see are never loaded
// ("BlockAttention" section: off-window tiles are skipped).
//
// Work decomposition. A persistent grid pops (sequence, query-tile, head) items,
// longest first, from the list ja_sched.hip built on the device. Each workgroup
// has four waves.
//   * Standard layout: the item is a 128-row query tile; wave w owns rows
//     [32w, 32w+32) and all four waves share each 64-key stage in LDS.
//   * Split layout (short queries, e.g. pooled attention with 32 seeds): the item
//     is a 32-row query tile; the waves split each 128-key stage four ways and
//     merge their partial results through LDS at the end.
//
// Per wave and 32-key block the scores are computed transposed, S^T = K Q^T, on
// the 32x32 matrix cores: A = K rows from LDS, B = the wave's queries held in
// registers for the whole item. In the C layout each lane then owns one query
// column, so the softmax statistics are per-lane scalars and a row reduction is a
// 16-register loop plus one exchange between the two half-waves. The probabilities
// P^T are already in the B-operand layout of the second product O^T += V^T P^T, so
// they feed it without any data movement; V is stored transposed in LDS (and keys
// are permuted inside the block, see key_of_arow) so that each lane's A operand is
// one contiguous vector read.
//
// K/V stages are double-buffered: the next stage is fetched from HBM into
// registers (coalesced 16-byte loads, zero-filled past the sequence end) while the
// current one is consumed, then written to the other LDS buffer; one barrier per
// stage. Masks are evaluated only on stages that cross the sequence end, the
// causal diagonal or a window edge; fully invisible blocks are skipped per wave.
// Softmax rescaling is lazy: the running max is only raised when a block exceeds
// it by more than 2^8, which leaves the result unchanged in exact arithmetic.
#include <math.h>

#include "ja_common.h"
#include "ja_internal.h"
#include "ja_tiles.h"

namespace ja {
namespace {

template <typename T, int D, bool SPLIT>
struct FwdCfg {
    static constexpr int NW = 4;                    // waves per workgroup
    static constexpr int WQ = SPLIT ? 1 : 4;        // query slices
    static constexpr int WK = NW / WQ;              // key slices
    static constexpr int NB = SPLIT ? 1 : 2;        // 32-key blocks per wave per stage
    static constexpr int BM = 32 * WQ;              // query rows per item
    static constexpr int KT = 32 * NB * WK;         // keys per stage
    static constexpr int KP = Mma<T>::KPACK;
    static constexpr int NS = D / (2 * KP);         // k-steps of S^T over d
    static constexpr int NT = 32 / (2 * KP);        // k-steps of P V over one 32-key block
    static constexpr int ND = D / 32;               // 32-row blocks of O^T
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int PAD = 16 / ESZ;            // 16 bytes of padding per LDS row
    static constexpr int KPITCH = D + PAD;          // K stored [key][d]
    static constexpr int VPITCH = KT + PAD;         // V stored transposed [d][key]
    static constexpr int K_ELEMS = KT * KPITCH;
    static constexpr int V_ELEMS = D * VPITCH;
    static constexpr int STAGE_BYTES = (K_ELEMS + V_ELEMS) * ESZ;
    static constexpr int VEC = 16 / ESZ;            // elements per 16-byte access
    static constexpr int KLOADS = KT * D / VEC / 256;
    static constexpr int VUNITS = (KT / 4) * (D / VEC);  // (4 keys x VEC dims) V units
    static constexpr int VLOADS = (VUNITS + 255) / 256;
    static constexpr int COMBINE_BYTES = SPLIT ? WK * 64 * (D / 2 + 2) * 4 : 0;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES > COMBINE_BYTES ? 2 * STAGE_BYTES : COMBINE_BYTES;
    static_assert(KT * D % (VEC * 256) == 0, "K stage must split evenly over 256 threads");
    static_assert(D % (2 * KP) == 0 && D % 32 == 0, "unsupported head dim");
};

template <typename T> struct Frag;
template <> struct Frag<bf16> {
    typedef bf16x8 type;
    static __device__ __forceinline__ type zero() { return type{}; }
};
template <> struct Frag<float> {
    typedef float type;
    static __device__ __forceinline__ type zero() { return 0.0f; }
};

// Pack four keys' VEC-element rows into VEC transposed groups of four keys.
template <typename T> struct VTrans;
template <> struct VTrans<bf16> {
    // r[i] holds 8 bf16 of key i; writes 8 x (4 keys) = 8 x 8 bytes.
    static __device__ __forceinline__ void store(bf16* dst, int pitch, const u32x4 r[4]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            u32x2 p;
            p[0] = __builtin_amdgcn_perm(r[1][e >> 1], r[0][e >> 1], sel);
            p[1] = __builtin_amdgcn_perm(r[3][e >> 1], r[2][e >> 1], sel);
            *(u32x2*)(dst + e * pitch) = p;
        }
    }
};
template <> struct VTrans<float> {
    static __device__ __forceinline__ void store(float* dst, int pitch, const u32x4 r[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u32x4 p;
            p[0] = r[0][e];
            p[1] = r[1][e];
            p[2] = r[2][e];
            p[3] = r[3][e];
            *(u32x4*)(dst + e * pitch) = p;
        }
    }
};

__device__ __forceinline__ bool visible(int row, int key, int Lk, int causal, int window) {
    if (key >= Lk) return false;
    if (causal && key > row) return false;
    if (window > 0) {
        int diff = row - key;
        if (!causal && diff < 0) diff = -diff;
        if (diff >= window) return false;
    }
    return true;
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

template <typename T, int D, int ACT, bool SPLIT>
__global__ __launch_bounds__(256) void ja_fwd_kernel(FwdArgs a) {
    using C = FwdCfg<T, D, SPLIT>;
    using M = Mma<T>;
    typedef typename Frag<T>::type frag;
    constexpr int KP = C::KP;

    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wq = SPLIT ? 0 : wave;
    const int wk = SPLIT ? wave : 0;
    const int col = lane & 31, grp = lane >> 5;
    const int total = a.counters[kCtrTotal];
    const T* __restrict__ Qg = (const T*)a.q;
    const T* __restrict__ Kg = (const T*)a.k;
    const T* __restrict__ Vg = (const T*)a.v;
    T* __restrict__ Og = (T*)a.out;
    const int64_t rs = (int64_t)a.H * D;  // token row stride, elements
    const int causal = a.causal, window = a.window;

    // Softmax works in the exp2 domain. With scale > 0 the row max is taken on raw
    // scores and folded into one FMA per element; otherwise scores are scaled first.
    const bool prescale = !(a.scale > 0.0f);
    const float c_exp = prescale ? 1.0f : a.scale * kLog2e;

    const int k_arow = key_of_arow<KP>(col);  // this lane's K row inside a 32-key block

    for (;;) {
        __syncthreads();
        if (tid == 0) s_item = atomicAdd(&a.counters[kCtrPop], 1);
        __syncthreads();
        const int idx = s_item;
        if (idx >= total) break;
        const int pair = idx / a.H, h = idx - pair * a.H;
        const int b = a.items[2 * pair], qt = a.items[2 * pair + 1];
        const int64_t qo = a.q_off[b], ko = a.k_off[b];
        // Rows are clamped to the tensors, so inconsistent offsets cannot reach
        // outside them (the header leaves such offsets undefined otherwise).
        const int Lq = qo < 0 ? 0 : min(a.q_off[b + 1], a.Tq) - (int)qo;
        const int Lk = ko < 0 ? 0 : min(a.k_off[b + 1], a.Tk) - (int)ko;
        const int q0 = qt * C::BM;
        const ColRange cr = visible_cols(Lq, Lk, q0, C::BM, causal, window, 0);
        const int kt_lo = cr.hi > cr.lo ? (int)(cr.lo / C::KT) : 0;
        const int kt_hi = cr.hi > cr.lo ? (int)((cr.hi + C::KT - 1) / C::KT) : 0;
        const int qw0 = q0 + 32 * wq;  // first query row of this wave
        const int my_row = qw0 + col;

        const T* Kseq = Kg + ko * rs + (int64_t)h * D;
        const T* Vseq = Vg + ko * rs + (int64_t)h * D;

        // Queries as the B operand of S^T = K Q^T, kept in registers.
        frag qf[C::NS];
        {
            const bool ok = my_row < Lq;
            const T* src = Qg + (qo + my_row) * rs + (int64_t)h * D + KP * grp;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) qf[s] = ok ? *(const frag*)(src + 2 * KP * s) : Frag<T>::zero();
        }

        floatx16 oacc[C::ND];
#pragma unroll
        for (int i = 0; i < C::ND; ++i) oacc[i] = floatx16{};
        float m_run = -INFINITY, l_run = 0.0f;

        u32x4 kr[C::KLOADS];
        u32x4 vr[C::VLOADS][4];

        auto issue = [&](int kt) {
            const int kbase = kt * C::KT;
            const int nvalid = Lk - kbase;
#pragma unroll
            for (int i = 0; i < C::KLOADS; ++i) {
                const int chunk = i * 256 + tid;
                const int key = chunk / (D / C::VEC), c = chunk % (D / C::VEC);
                kr[i] = key < nvalid ? *(const u32x4*)(Kseq + (int64_t)(kbase + key) * rs + c * C::VEC)
                                     : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < C::VLOADS; ++j) {
                const int u = j * 256 + tid;
                const int kg = u % (C::KT / 4), dc = u / (C::KT / 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 4 * kg + i;
                    vr[j][i] = (u < C::VUNITS && key < nvalid)
                                   ? *(const u32x4*)(Vseq + (int64_t)(kbase + key) * rs + dc * C::VEC)
                                   : u32x4{0u, 0u, 0u, 0u};
                }
            }
        };
        auto store = [&](int buf) {
            T* kl = (T*)(smem + buf * C::STAGE_BYTES);
            T* vl = kl + C::K_ELEMS;
#pragma unroll
            for (int i = 0; i < C::KLOADS; ++i) {
                const int chunk = i * 256 + tid;
                const int key = chunk / (D / C::VEC), c = chunk % (D / C::VEC);
                *(u32x4*)(kl + key * C::KPITCH + c * C::VEC) = kr[i];
            }
#pragma unroll
            for (int j = 0; j < C::VLOADS; ++j) {
                const int u = j * 256 + tid;
                if (u < C::VUNITS) {
                    const int kg = u % (C::KT / 4), dc = u / (C::KT / 4);
                    VTrans<T>::store(vl + (dc * C::VEC) * C::VPITCH + 4 * kg, C::VPITCH, vr[j]);
                }
            }
        };

        if (kt_hi > kt_lo) {
            issue(kt_lo);
            store(0);
            __syncthreads();
        }

        for (int kt = kt_lo; kt < kt_hi; ++kt) {
            const int buf = (kt - kt_lo) & 1;
            const bool more = kt + 1 < kt_hi;
            if (more) issue(kt + 1);

            const T* kl = (const T*)(smem + buf * C::STAGE_BYTES);
            const T* vl = kl + C::K_ELEMS;
            const int kw0 = kt * C::KT + wk * 32 * C::NB;  // first key of this wave's blocks
            const bool skip = qw0 >= Lq || block_all_masked(qw0, 32, kw0, 32 * C::NB, Lk, causal, window);
            if (!skip) {
                floatx16 sacc[C::NB];
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    sacc[nb] = floatx16{};
                    const T* krow = kl + (wk * 32 * C::NB + nb * 32 + k_arow) * C::KPITCH + KP * grp;
#pragma unroll
                    for (int s = 0; s < C::NS; ++s)
                        sacc[nb] = M::run(*(const frag*)(krow + 2 * KP * s), qf[s], sacc[nb]);
                }

                const bool need_mask = block_needs_mask(qw0, 32, kw0, 32 * C::NB, Lk, causal, window);
                uint32_t vis = 0xffffffffu;  // bit nb*16+r: element visible
                if (need_mask) {
                    vis = 0;
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kw0 + nb * 32 + key_of_reg<KP>(grp, r);
                            if (visible(my_row, key, Lk, causal, window)) vis |= 1u << (nb * 16 + r);
                        }
                }

                if (ACT == ACT_SOFTMAX) {
                    if (prescale) {
#pragma unroll
                        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) sacc[nb][r] *= a.scale * kLog2e;
                    }
                    if (need_mask) {
#pragma unroll
                        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                if (!(vis >> (nb * 16 + r) & 1u)) sacc[nb][r] = -INFINITY;
                    }
                    float mx = -INFINITY;
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
                    mx = xhalf_max(mx) * c_exp;
                    if (__any(mx > m_run + 8.0f)) {
                        const float m_new = fmaxf(m_run, mx);
                        const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_run - m_new);
                        l_run *= alpha;
#pragma unroll
                        for (int i = 0; i < C::ND; ++i) oacc[i] *= alpha;
                        m_run = m_new;
                    }
                    const float msub = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float p = fast_exp2(fmaf(sacc[nb][r], c_exp, -msub));
                            l_run += p;
                            sacc[nb][r] = p;
                        }
                } else {
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            float p = pointwise<ACT>(sacc[nb][r] * a.scale);
                            if (need_mask && !(vis >> (nb * 16 + r) & 1u)) p = 0.0f;
                            sacc[nb][r] = p;
                        }
                }

                // P^T in the B-operand layout, then O^T += V^T P^T.
                frag pf[C::NB][C::NT];
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                    for (int t = 0; t < C::NT; ++t) {
                        if constexpr (KP == 8) {
#pragma unroll
                            for (int s = 0; s < 8; ++s) pf[nb][t][s] = (bf16)sacc[nb][8 * t + s];
                        } else {
                            pf[nb][t] = sacc[nb][t];
                        }
                    }
#pragma unroll
                for (int db = 0; db < C::ND; ++db) {
                    const T* vrow = vl + (32 * db + col) * C::VPITCH + wk * 32 * C::NB + KP * grp;
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                        for (int t = 0; t < C::NT; ++t)
                            oacc[db] = M::run(*(const frag*)(vrow + nb * 32 + 2 * KP * t), pf[nb][t], oacc[db]);
                }
            }

            if (more) store(buf ^ 1);
            __syncthreads();
        }

        // Split layout: merge the four key slices through LDS (stage buffers are
        // free: the loop ended on a barrier, or no stage was loaded at all).
        if constexpr (SPLIT) {
            float* red_o = (float*)smem;                  // [wave][D/2][64]
            float* red_m = red_o + C::WK * (D / 2) * 64;  // [wave][64]
            float* red_l = red_m + C::WK * 64;            // [wave][64]
            if (ACT == ACT_SOFTMAX) {
                red_m[wave * 64 + lane] = m_run;
                __syncthreads();
                float mg = -INFINITY;
#pragma unroll
                for (int w = 0; w < C::WK; ++w) mg = fmaxf(mg, red_m[w * 64 + lane]);
                const float sc = m_run == -INFINITY ? 0.0f : fast_exp2(m_run - mg);
                l_run *= sc;
#pragma unroll
                for (int i = 0; i < C::ND; ++i) oacc[i] *= sc;
                m_run = mg;
            }
            if (wave > 0) {
                red_l[wave * 64 + lane] = l_run;
#pragma unroll
                for (int i = 0; i < C::ND; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red_o[((wave * C::ND + i) * 16 + r) * 64 + lane] = oacc[i][r];
            }
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int w = 1; w < C::WK; ++w) {
                    l_run += red_l[w * 64 + lane];
#pragma unroll
                    for (int i = 0; i < C::ND; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[i][r] += red_o[((w * C::ND + i) * 16 + r) * 64 + lane];
                }
            }
        }

        if (!SPLIT || wave == 0) {
            float inv;
            float lse_val = 0.0f;
            if (ACT == ACT_SOFTMAX) {
                const float l_tot = xhalf_sum(l_run);
                inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
                lse_val = l_tot > 0.0f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
            } else {
                inv = Lk > 0 ? 1.0f / (float)Lk : 0.0f;
            }
            if (my_row < Lq) {
                T* dst = Og + (qo + my_row) * rs + (int64_t)h * D + 4 * grp;
#pragma unroll
                for (int i = 0; i < C::ND; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        store4<T>(dst + 32 * i + 8 * j, oacc[i][4 * j] * inv, oacc[i][4 * j + 1] * inv,
                                  oacc[i][4 * j + 2] * inv, oacc[i][4 * j + 3] * inv);
                if (ACT == ACT_SOFTMAX && a.lse != nullptr && grp == 0)
                    a.lse[(qo + my_row) * a.H + h] = lse_val;
            }
        }
    }
}

template <typename T, int D, int ACT, bool SPLIT>
struct FwdKernel {
    static void* fn() { return (void*)ja_fwd_kernel<T, D, ACT, SPLIT>; }
};

template <typename T, int D, int ACT, bool SPLIT>
hipError_t launch_one(const FwdArgs& a, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((ja_fwd_kernel<T, D, ACT, SPLIT>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D, int ACT, bool SPLIT>
int occupancy_one() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ja_fwd_kernel<T, D, ACT, SPLIT>, 256, 0) != hipSuccess)
        return 1;
    return n > 0 ? n : 1;
}

// Dispatch over (dtype, d, act, split) to a callable template F<T, D, ACT, SPLIT>.
template <template <typename, int, int, bool> class F, typename R, typename... Args>
R dispatch(int dtype, int d, int act, bool split, R fail, Args... args) {
#define JA_ACTS(T, D, S)                                              \
    switch (act) {                                                    \
        case ACT_SOFTMAX: return F<T, D, ACT_SOFTMAX, S>::call(args...); \
        case ACT_SILU: return F<T, D, ACT_SILU, S>::call(args...);       \
        case ACT_GELU: return F<T, D, ACT_GELU, S>::call(args...);       \
        default: return fail;                                         \
    }
#define JA_DIMS(T, S)                      \
    switch (d) {                           \
        case 32: JA_ACTS(T, 32, S)         \
        case 64: JA_ACTS(T, 64, S)         \
        case 128: JA_ACTS(T, 128, S)       \
        default: return fail;              \
    }
    if (dtype == 1) {
        if (split) { JA_DIMS(bf16, true) }
        JA_DIMS(bf16, false)
    }
    if (dtype == 0) { JA_DIMS(float, false) }
#undef JA_DIMS
#undef JA_ACTS
    return fail;
}

template <typename T, int D, int ACT, bool SPLIT>
struct LaunchF {
    static hipError_t call(const FwdArgs* a, int grid, hipStream_t s) { return launch_one<T, D, ACT, SPLIT>(*a, grid, s); }
};
template <typename T, int D, int ACT, bool SPLIT>
struct OccF {
    static int call() { return occupancy_one<T, D, ACT, SPLIT>(); }
};
template <typename T, int D, int ACT, bool SPLIT>
struct ShapeF {
    static FwdShape call() { return FwdShape{FwdCfg<T, D, SPLIT>::BM, FwdCfg<T, D, SPLIT>::KT}; }
};

}  // namespace

bool fwd_supported(int dtype, int d, int act) {
    return (dtype == 0 || dtype == 1) && (d == 32 || d == 64 || d == 128) && act >= 0 && act <= 2;
}

FwdShape fwd_shape(int dtype, int d, int act, bool split) {
    return dispatch<ShapeF, FwdShape>(dtype, d, act, split && dtype == 1, FwdShape{0, 0});
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int d, int act, bool split, int grid, hipStream_t stream) {
    return dispatch<LaunchF, hipError_t>(dtype, d, act, split && dtype == 1, hipErrorInvalidValue, &a, grid,
                                         stream);
}

int fwd_blocks_per_cu(int dtype, int d, int act, bool split) {
    return dispatch<OccF, int>(dtype, d, act, split && dtype == 1, 1);
}

}  // namespace ja
