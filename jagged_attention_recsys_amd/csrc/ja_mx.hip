// ja_mx.hip -- MXFP8 jagged attention forward for gfx950, and its quantizer.
//
// "Mixed Ultra-Low-Precision Training" section of the GEM training post: the
// attention's matrix products run on block-scaled FP8 (MXFP8) with one scale per
// [32, 32] block, so that a tensor and its transpose share one quantization, and
// the softmax weights P are quantized online, their scale set by the softmax's
// own row max. Format (OCP MX): E4M3 elements ("fn": largest finite 448), E8M0
// power-of-two scales. A block is 32 consecutive tokens of one sequence (blocks
// restart at every sequence start) by 32 channels of one head; its scale
// exponent is floor(log2(amax)) - 8, limited to [-127, 127], and each element is
// x / 2^e clamped to +-448 and rounded to nearest even.
//
// Forward: the general forward's standard layout (4 waves, 128-row query tiles,
// 64-key stages double-buffered through LDS by buffer loads, persistent grid
// over the device-built longest-first list) on v_mfma_scale_f32_32x32x64_f8f6f4:
//   S^T = K Q^T, two products per 32-key block over d = 128, with the K and Q
//   block scales as the instruction's per-lane scales;
//   softmax with a lazy running max (raised only when a block exceeds it by more
//   than kMxLazy = 0.75 in the exp2 domain), so every weight p = exp2(s - m) is at
//   most 2^0.75 and, rounded to E4M3 at the fixed scale 2^-8, at most 430 of the
//   format's 448 (no per-block amax: the running max already bounds it); most
//   stages then skip the rescale of the accumulators;
//   O^T += V^T P^T, one product per 32-channel block over all 64 keys, V^T read
//   from V's natural layout by 8-bit LDS transpose reads, V's block scales per
//   lane.
// Operand layout of the 32x32x64 instruction (probed in bounds on the GPU): lane
// (i, g) of A holds row i, its bytes 0-15 the k slots 16g..16g+15 and bytes
// 16-31 the slots 32+16g..32+16g+15; B likewise with columns; the scale of lane
// (i, g) covers k slots [32g, 32g + 32). K rows are permuted inside each 32-key
// block (A row slot i holds key 16((i>>2)&1) + 4(i>>3) + (i&3)) so that lane g of
// S^T's C tile holds keys 16g..16g+15 in register order: those are exactly the
// P^T bytes the second product needs, with no data movement.
#include <math.h>

#include "ja_common.h"
#include "ja_internal.h"
#include "ja_lds.h"
#include "ja_mx.h"
#include "ja_tiles.h"

namespace ja {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMxWaves = 4;
constexpr int kMxThreads = 64 * kMxWaves;
constexpr int kMxRowB = kMxD;              // bytes per FP8 row of one head
[[maybe_unused]] constexpr int kMxTile = kMxKT * kMxRowB;  // one K or V stage
[[maybe_unused]] constexpr int kMxNKB = kMxKT / 32;          // 32-key blocks per stage
[[maybe_unused]] constexpr int kMxNKH = kMxKT / 64;          // 64-key halves per stage (one P V product each)
[[maybe_unused]] constexpr int kMxLPW = kMxTile / 1024 / kMxWaves;  // 64-lane loads per wave per tile
[[maybe_unused]] constexpr int kPScale = 127 - 8;          // E8M0 scale 2^-8 of the quantized softmax weights
// Slack of the running max (exp2 domain): 2^(8 + kMxLazy) = 430.5 stays below E4M3's
// largest finite value, 448 = 2^8 * 1.75, with room for the fp32 rounding of the
// exponent's argument.
[[maybe_unused]] constexpr float kMxLazy = 0.75f;

#if defined(__HIP_DEVICE_COMPILE__)
// Floor of log2 of a positive finite float, exact for subnormals too.
__device__ __forceinline__ int floor_log2(float a) {
    const uint32_t u = __float_as_uint(a);
    const int e = (int)((u >> 23) & 0xff);
    if (e != 0) return e - 127;
    return (31 - __clz(u & 0x7fffff)) - 149;
}

// E8M0 exponent of a block with largest magnitude amax.
__device__ __forceinline__ int mx_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    const int e = floor_log2(amax) - 8;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four floats (already scaled, within +-448) to four E4M3 codes, nearest even.
// The first conversion writes the low half, the second the high half, so the
// word the first one starts from is irrelevant (a's own bits: no extra move).
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)__float_as_uint(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }
#endif

// ---- quantizer ------------------------------------------------------------

// One workgroup: first block of every sequence (prefix of ceil(L/32)) and the
// sequence of every block.
__global__ __launch_bounds__(1024) void ja_mx_prefix_kernel(MxQuantArgs a) {
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    const int chunk = (a.B + 1023) / 1024;
    const int b0 = min(a.B, t * chunk), b1 = min(a.B, b0 + chunk);
    int32_t sum = 0;
    for (int b = b0; b < b1; ++b) {
        const int L = max(0, min(a.off[b + 1], a.T) - max(a.off[b], 0));
        sum += (L + kMxBlock - 1) / kMxBlock;
    }
    part[t] = sum;
    __syncthreads();
    if (t == 0) {
        int32_t run = 0;
        for (int i = 0; i < 1024; ++i) {
            const int32_t v = part[i];
            part[i] = run;
            run += v;
        }
        a.soff[a.B] = run;
    }
    __syncthreads();
    int32_t base = part[t];
    for (int b = b0; b < b1; ++b) {
        a.soff[b] = base;
        const int L = max(0, min(a.off[b + 1], a.T) - max(a.off[b], 0));
        const int nb = (L + kMxBlock - 1) / kMxBlock;
        for (int j = 0; j < nb; ++j)
            if (base + j < a.max_blocks) a.blk_seq[base + j] = b;
        base += nb;
    }
}

// One workgroup per 32-token block; each wave takes (head, 32-channel) blocks,
// lane l covering token l/2 and 16 channels.
__global__ __launch_bounds__(256) void ja_mx_quant_kernel(MxQuantArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int jb = blockIdx.x;
    const int nblocks = min(a.soff[a.B], a.max_blocks);
    if (jb >= nblocks) return;
    const int b = a.blk_seq[jb];
    const int64_t r0 = a.off[b] + (int64_t)(jb - a.soff[b]) * kMxBlock;
    const int rows = min(kMxBlock, min(a.off[b + 1], a.T) - (int)r0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane >> 1, half = lane & 1;
    const int nd = a.d / kMxBlock;
    for (int pc = wave; pc < a.H * nd; pc += 4) {
        const int h = pc / nd, c = pc - h * nd;
        const int64_t e0 = ((r0 + row) * a.H + h) * a.d + c * kMxBlock + 16 * half;
        float v[16];
        const bool ok = row < rows;
        {
            const bf16x8* src = (const bf16x8*)((const bf16*)a.x + e0);
            const bf16x8 lo = ok ? src[0] : bf16x8{};
            const bf16x8 hi = ok ? src[1] : bf16x8{};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[i] = (float)lo[i];
                v[8 + i] = (float)hi[i];
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const int ex = mx_exponent(amax);
        const float mul = __uint_as_float((uint32_t)(127 - ex) << 23);  // 2^-ex, a normal float here
        if (lane == 0) a.scales[((int64_t)jb * a.H + h) * nd + c] = (uint8_t)(ex + 127);
        if (ok) {
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = pack4(clamp448(v[4 * q] * mul), clamp448(v[4 * q + 1] * mul), clamp448(v[4 * q + 2] * mul),
                             clamp448(v[4 * q + 3] * mul));
            *(u32x4*)(a.x8 + e0) = w;
        }
    }
#else
    (void)a;
#endif
}

// ---- attention forward ------------------------------------------------------
#if defined(__HIP_DEVICE_COMPILE__)
// XOR swizzle of the 16-byte chunks of a 128-byte FP8 row: the operand reads of
// K (16 lanes, 16 rows, one chunk) and the transpose reads of V (32 lanes, 8
// rows, two chunks) both hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int row) { return (((row >> 1) & 3) << 1) | ((row >> 4) & 1); }

// Key held by A row slot i of a 32-key block: lane g of the C tile then holds
// keys 16g..16g+15 in register order.
__device__ __forceinline__ int key_of_slot(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i read_k(const char* blk, int o0, int o1) {
    const i32x4 lo = *(const i32x4*)(blk + o0);
    const i32x4 hi = *(const i32x4*)(blk + o1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ v2i read_tr8(const char* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)p);
}
#endif

__global__ __launch_bounds__(kMxThreads, 2) void ja_mx_fwd_kernel(MxFwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    __shared__ __attribute__((aligned(1024))) char lds_k0[kMxTile];
    __shared__ __attribute__((aligned(1024))) char lds_v0[kMxTile];
    __shared__ __attribute__((aligned(1024))) char lds_k1[kMxTile];
    __shared__ __attribute__((aligned(1024))) char lds_v1[kMxTile];
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, g = lane >> 5;
    const int total = a.counters[kCtrTotal];
    const int64_t rs = (int64_t)a.H * kMxD;   // bytes per token row
    const uint32_t rsb = (uint32_t)rs;
    const int causal = a.causal, window = a.window;
    const bool prescale = !(a.scale > 0.0f);
    const float c_exp = prescale ? 1.0f : a.scale * kLog2e;

    // Stage loads: slot (wave + 4j) * 64 + lane of a tile is chunk p of row r.
    uint32_t voff[kMxLPW];
#pragma unroll
    for (int j = 0; j < kMxLPW; ++j) {
        const int slot = (wave + j * kMxWaves) * 64 + lane;
        const int r = slot >> 3, p = slot & 7;
        voff[j] = (uint32_t)r * rsb + (uint32_t)((p ^ swz8(r)) << 4);
    }
    // K operand reads: row key_of_slot(col), chunks 4c + g and 4c + 2 + g.
    int koff[2][2];
    {
        const int r = key_of_slot(col);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            koff[c][0] = r * kMxRowB + (((4 * c + g) ^ swz8(r)) << 4);
            koff[c][1] = r * kMxRowB + (((4 * c + 2 + g) ^ swz8(r)) << 4);
        }
    }
    // V transpose reads: 16-lane group G reads, for 32-channel block db, rows
    // rb + 0..7 at channels 32db + 16(G & 1) + 0..15, rb = 32(j>>1) + 16g + 8(j&1).
    int toff[4][4];
    {
        const int i16 = lane & 15, G = lane >> 4;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 32 * (j >> 1) + 16 * g + 8 * (j & 1) + (i16 >> 1);
                const int ch = 32 * db + 16 * (G & 1) + 8 * (i16 & 1);
                toff[db][j] = r * kMxRowB + (((ch >> 4) ^ swz8(r)) << 4) + (ch & 15);
            }
    }

    // Waits for LDS operations only: no buffer-to-LDS stage load is outstanding at
    // an item boundary (each item's stages are consumed before its last stage
    // barrier, a __syncthreads that waits for every vector memory operation).
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    int next = 0;
    if (tid == 0) next = atomicAdd(&a.counters[kCtrPop], 1);
    for (;;) {
        if (tid == 0) s_item = next;
        lds_barrier();
        const int idx = __builtin_amdgcn_readfirstlane(s_item);
        lds_barrier();
        if (idx >= total) break;
        const int pair = idx / a.H, h = idx - pair * a.H;
        const ItemSeq is = load_item(a.items, pair, false, a.Tq, a.Tk);
        const int b = is.b, qt = is.t;
        const int64_t qo = is.qo, ko = is.ko;
        const int Lq = is.Lq, Lk = is.Lk;
        const int q0 = qt * kMxBM;
        const ColRange cr = visible_cols(Lq, Lk, q0, kMxBM, causal, window, 0, kNoBlock);
        const int kt_lo = cr.hi > cr.lo ? (int)(cr.lo / kMxKT) : 0;
        const int kt_hi = cr.hi > cr.lo ? (int)((cr.hi + kMxKT - 1) / kMxKT) : 0;
        const int qw0 = q0 + 32 * wave;
        const int my_row = qw0 + col;
        const bool row_ok = my_row < Lq;
        const VisRange vis = keys_seen_by(my_row, Lk, causal, window, kNoBlock);
        const int nkblk = (Lk + kMxBlock - 1) / kMxBlock;  // scale blocks of this sequence's keys

        // Q as B operands (two k-halves of d) and their block scales.
        v8i qf[2];
        int qsc[2];
        {
            const char* src = (const char*)a.q8 + (qo + my_row) * rs + (int64_t)h * kMxD;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const u32x4 lo = row_ok ? *(const u32x4*)(src + 64 * c + 16 * g) : u32x4{};
                const u32x4 hi = row_ok ? *(const u32x4*)(src + 64 * c + 32 + 16 * g) : u32x4{};
                qf[c] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
            const uint32_t w = qw0 < Lq
                ? *(const uint32_t*)(a.qs + ((int64_t)(a.q_soff[b] + (qw0 >> 5)) * a.H + h) * 4)
                : 0x7f7f7f7fu;
#pragma unroll
            for (int c = 0; c < 2; ++c) qsc[c] = (int)((w >> (8 * (2 * c + g))) & 0xff);
        }

        floatx16 oacc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[i] = floatx16{};
        float m_run = -INFINITY, l_run = 0.0f;

        const char* Kseq = (const char*)a.k8 + ko * rs + (int64_t)h * kMxD;
        const char* Vseq = (const char*)a.v8 + ko * rs + (int64_t)h * kMxD;
        const int64_t kblk0 = a.k_soff[b];

        // Stage kt: K and V rows [KT kt, KT kt + KT) into LDS; the K scale words of
        // its key blocks and the V scale words of this lane's key block in each
        // 64-key half.
        auto issue = [&](int kt, char* kdst, char* vdst, uint32_t (&ksw)[kMxNKB], uint32_t (&vsw)[kMxNKH]) {
            const int kbase = kt * kMxKT;
            const uint32_t nrec = __builtin_amdgcn_readfirstlane((uint32_t)min(max(Lk - kbase, 0), kMxKT) * rsb);
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc((void*)(Kseq + (int64_t)kbase * rsb), (short)0, (int)nrec, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void*)(Vseq + (int64_t)kbase * rsb), (short)0, (int)nrec, 0x00020000);
#pragma unroll
            for (int j = 0; j < kMxLPW; ++j) {
                const int inst = wave + j * kMxWaves;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_char*)kdst + inst * 1024, 16, voff[j], 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_char*)vdst + inst * 1024, 16, voff[j], 0, 0, 0);
            }
#pragma unroll
            for (int nb = 0; nb < kMxNKB; ++nb) {
                const int kb = kMxNKB * kt + nb;
                ksw[nb] = kb < nkblk ? *(const uint32_t*)(a.ks + ((kblk0 + kb) * a.H + h) * 4) : 0x7f7f7f7fu;
            }
#pragma unroll
            for (int kh = 0; kh < kMxNKH; ++kh) {
                const int vb = kMxNKB * kt + 2 * kh + g;
                vsw[kh] = vb < nkblk ? *(const uint32_t*)(a.vs + ((kblk0 + vb) * a.H + h) * 4) : 0x7f7f7f7fu;
            }
        };

        auto stage = [&](int kt, const char* kl, const char* vl, char* kn, char* vn,
                         const uint32_t (&ksc)[kMxNKB], const uint32_t (&vsc)[kMxNKH], uint32_t (&ksn)[kMxNKB],
                         uint32_t (&vsn)[kMxNKH]) {
            if (kt + 1 < kt_hi) issue(kt + 1, kn, vn, ksn, vsn);
            const int kw0 = kt * kMxKT;
            const bool skip = wave_skips(vis, row_ok, kw0, kMxKT);
            if (!skip) {
                // Matrix operands are read from LDS ahead of their products (K two
                // products ahead; V's first two before the weights, whose vector work
                // hides their latency): left to itself the compiler reads each operand
                // next to its product and waits for it every time.
                constexpr int NSK = kMxNKB * 2, RK = 2, NPV = kMxNKH * 4, RV = 2;
                auto kread = [&](int i) __attribute__((always_inline)) {
                    return read_k(kl + (i >> 1) * 32 * kMxRowB, koff[i & 1][0], koff[i & 1][1]);
                };
                auto vread = [&](int i) __attribute__((always_inline)) {
                    const char* vh = vl + (i >> 2) * 64 * kMxRowB;
                    const int db = i & 3;
                    const i32x4 t01 = __builtin_shufflevector(read_tr8(vh + toff[db][0]), read_tr8(vh + toff[db][1]),
                                                              0, 1, 2, 3);
                    const i32x4 t23 = __builtin_shufflevector(read_tr8(vh + toff[db][2]), read_tr8(vh + toff[db][3]),
                                                              0, 1, 2, 3);
                    return (v8i)__builtin_shufflevector(t01, t23, 0, 1, 2, 3, 4, 5, 6, 7);
                };
                floatx16 sacc[kMxNKB];
#pragma unroll
                for (int nb = 0; nb < kMxNKB; ++nb) sacc[nb] = floatx16{};
                v8i kr[RK];
#pragma unroll
                for (int i = 0; i < RK; ++i) kr[i] = kread(i);
#pragma unroll
                for (int i = 0; i < NSK; ++i) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int nb = i >> 1, c = i & 1;
                    const int ksb = (int)((ksc[nb] >> (8 * (2 * c + g))) & 0xff);
                    sacc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kr[i % RK], qf[c], sacc[nb], 0, 0, 0,
                                                                               ksb, 0, qsc[c]);
                    if (i + RK < NSK) kr[i % RK] = kread(i + RK);
                }
                __builtin_amdgcn_sched_barrier(0);
                v8i vr[RV];
#pragma unroll
                for (int i = 0; i < RV; ++i) vr[i] = vread(i);
                __builtin_amdgcn_sched_barrier(0);
                // Wave-uniform branches around whole loops (not a select per score).
                if (prescale) {
#pragma unroll
                    for (int nb = 0; nb < kMxNKB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) sacc[nb][r] *= a.scale * kLog2e;
                }
                if (wave_needs_mask(vis, row_ok, kw0, kMxKT)) {
#pragma unroll
                    for (int nb = 0; nb < kMxNKB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            sacc[nb][r] = vis.has(kw0 + nb * 32 + 16 * g + r) ? sacc[nb][r] : -INFINITY;
                }
                float mx = -INFINITY;
#pragma unroll
                for (int nb = 0; nb < kMxNKB; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
                mx = halves_max(mx) * c_exp;
                // Lazy running max: every weight below stays <= 2^kMxLazy.
                if (__any(mx > m_run + kMxLazy)) {
                    const float m_new = fmaxf(m_run, mx);
                    const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_run - m_new);
                    l_run *= alpha;
#pragma unroll
                    for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
                    m_run = m_new;
                }
                // Weights come out of the exponential already scaled by 2^8 (the E4M3
                // scale of P); the running sum carries the same factor.
                const float msub = (m_run == -INFINITY ? 0.0f : m_run) - 8.0f;
                float lsum[4];
                v8i pf[kMxNKH];
#pragma unroll
                for (int nb = 0; nb < kMxNKB; ++nb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float p4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float p = fast_exp2(fmaf(sacc[nb][4 * q + e], c_exp, -msub));
                            lsum[e] = (nb == 0 && q == 0) ? p : lsum[e] + p;
                            p4[e] = p;
                        }
                        pf[nb >> 1][4 * (nb & 1) + q] = (int)pack4(p4[0], p4[1], p4[2], p4[3]);
                    }
                l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
#pragma unroll
                for (int i = 0; i < NPV; ++i) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int kh = i >> 2, db = i & 3;
                    const int vsb = (int)((vsc[kh] >> (8 * db)) & 0xff);
                    oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vr[i % RV], pf[kh], oacc[db], 0, 0, 0,
                                                                                vsb, 0, kPScale);
                    if (i + RV < NPV) vr[i % RV] = vread(i + RV);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
        };

        uint32_t ks0[kMxNKB], ks1[kMxNKB], vs0[kMxNKH], vs1[kMxNKH];
#pragma unroll
        for (int i = 0; i < kMxNKB; ++i) ks0[i] = ks1[i] = 0;
#pragma unroll
        for (int i = 0; i < kMxNKH; ++i) vs0[i] = vs1[i] = 0;
        if (kt_hi > kt_lo) {
            issue(kt_lo, lds_k0, lds_v0, ks0, vs0);
            __syncthreads();
        }
        for (int kt = kt_lo; kt < kt_hi; kt += 2) {
            stage(kt, lds_k0, lds_v0, lds_k1, lds_v1, ks0, vs0, ks1, vs1);
            if (kt + 1 < kt_hi) stage(kt + 1, lds_k1, lds_v1, lds_k0, lds_v0, ks1, vs1, ks0, vs0);
        }

        if (tid == 0) next = atomicAdd(&a.counters[kCtrPop], 1);

        const float l_tot = halves_sum(l_run);  // 2^8 times the softmax normaliser
        const float inv = l_tot > 0.0f ? 256.0f / l_tot : 0.0f;
        {
            // Output rows written whole (16 bytes per lane) through the wave's half
            // of a second stage buffer, free after the stage loop's last barrier.
            using RT = RowTurn<kMxD>;
            static_assert(2 * RT::BYTES <= kMxTile, "two wave regions per stage array");
            char* const wreg = (wave < 2 ? lds_k1 : lds_v1) + (wave & 1) * RT::BYTES;
            RT::put_acc(wreg, oacc, inv, lane);
            RT::store((bf16*)a.out + (qo + qw0) * rs + (int64_t)h * kMxD, rs, Lq - qw0, wreg, lane);
        }
        if (row_ok) {
            if (a.lse != nullptr && g == 0)
                a.lse[(qo + my_row) * a.H + h] = l_tot > 0.0f ? (m_run - 8.0f) * kLn2 + logf(l_tot) : -INFINITY;
        }
    }
#else
    (void)a;
#endif
}

}  // namespace

hipError_t launch_mx_quant(const MxQuantArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(ja_mx_prefix_kernel, dim3(1), dim3(1024), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.max_blocks > 0) hipLaunchKernelGGL(ja_mx_quant_kernel, dim3(a.max_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_mx_fwd(const MxFwdArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL(ja_mx_fwd_kernel, dim3(grid), dim3(kMxThreads), 0, s, a);
    return hipGetLastError();
}

int mx_fwd_blocks_per_cu() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&ja_mx_fwd_kernel),
                                                     kMxThreads, 0) != hipSuccess)
        n = 1;
    return n > 0 ? n : 1;
}

}  // namespace ja
