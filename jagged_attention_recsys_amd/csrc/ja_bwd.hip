// ja_bwd.hip -- jagged attention backward for gfx950, split into a
// query-stationary dQ pass and a key-stationary dK/dV pass ("Jagged Sequence
// Flash Attention" section of the GEM training post: dQ in its own pass, no
// atomic accumulation of any gradient, no recomputation shared across passes).
//
// Softmax, with P = exp(scale Q K^T - lse) (the forward's log-sum-exp per row):
//   Di  = sum_c dO_ic O_ic                       (dQ pass prologue, to workspace)
//   dP  = dO V^T,  dS = P o (dP - Di)
//   dQ  = scale dS K                             (dQ pass, written once)
//   dV  = P^T dO,  dK = scale dS^T Q             (dK/dV pass, written once)
//
// Pointwise SiLU / tanh-GELU ("Generalized Dot-Product Attention (GDPA)"
// section: the activation replaces softmax, output normalised by 1/Lk), with
// Z = scale Q K^T: P = act(Z) / Lk and dS = act'(Z) o dP / Lk, then the same
// three products. There is no lse, no Di and no forward output to read.
//
// dQ pass: 4 waves, a 128-row query tile, wave w owns 32 rows. For each 64-key
// stage (K and V streamed into LDS as in the forward): S^T = K Q^T and
// dP^T = V dO^T on the matrix cores (queries and dO held as B operands in
// registers, so every lane owns one query column), then dQ^T += K^T dS^T with K^T
// read through LDS transpose reads.
//
// dK/dV pass: 4 waves, a 128-key tile, wave w owns 32 keys (K and V held as B
// operands). For each 64-query stage (Q, dO, -lse log2(e) and Di streamed into LDS):
// S = Q K^T and dP = dO V^T give lane-per-key C tiles; dV^T += dO^T P and
// dK^T += Q^T dS use transpose reads of dO and Q. Query tiles no key of the item
// can see (causal diagonal, window) are never loaded.
#include <math.h>

#include "ja_common.h"
#include "ja_internal.h"
#include "ja_lds.h"
#include "ja_tiles.h"

namespace ja {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRows = 32 * kBwdWaves;  // rows (queries or keys) per work item
constexpr int kBwdStage = 64;             // columns (keys or queries) per stage

template <typename T, int D>
struct BwdCfg {
    using STile = Tile<T, D, kBwdStage>;  // one stage of K, V, Q or dO
    using Loader = TileLoader<STile, kBwdWaves>;
    static constexpr int KP = STile::KP;
    static constexpr int NS = STile::NS;
    static constexpr int ND = STile::ND;
    static constexpr int NB = kBwdStage / 32;  // 32-column blocks per stage
    static constexpr int NT = 32 / (2 * KP);   // k-steps per 32-column block
    static constexpr int ROWB = STile::ROWB;
};

// dQ pass ---------------------------------------------------------------------
// The dQ pass fits in 256 VGPRs, so two of its workgroups share a CU; the dK/dV
// pass holds two accumulators per row and runs one workgroup per CU.
template <typename T, int D, int ACT, typename GT>
__global__ __launch_bounds__(kBwdThreads, 2) void ja_bwd_dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = BwdCfg<T, D>;
    using M = Mma<T>;
    typedef typename Frag<T>::type frag;
    constexpr int KP = C::KP;

    __shared__ __attribute__((aligned(1024))) char lds_k0[C::STile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v0[C::STile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_k1[C::STile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v1[C::STile::BYTES];
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, grp = lane >> 5;
    const int total = a.q_counters[kCtrTotal];
    const int64_t rs = (int64_t)a.H * D;
    const uint32_t rsb = (uint32_t)(rs * (int)sizeof(T));
    const int causal = a.causal, window = a.window, bsh = a.bsh;
    const float c_exp = a.scale * kLog2e;

    int koff[C::NS];
    int toff[C::ND][2];
    C::STile::row_offsets(col, grp, koff);
    C::STile::tr_offsets(lane, toff);
    typename C::Loader ld;
    ld.init(wave, lane, rsb);

    __shared__ int s_xq[2];
    int pend = 0;  // thread 0's pop in flight, sent before the previous item's output
    if (tid == 0) {
        xq_init(s_xq, a.window > 0);
        pend = xq_issue(a.q_counters, s_xq);
    }
    for (;;) {
        __syncthreads();
        if (tid == 0) s_item = xq_resolve(a.q_counters, s_xq, pend, total);
        __syncthreads();
        const int idx = __builtin_amdgcn_readfirstlane(s_item);
        if (idx >= total) break;
        const int pair = idx / a.H, h = idx - pair * a.H;
        const ItemSeq is = load_item(a.q_items, pair, false, a.Tq, a.Tk);
        const int qt = is.t;
        const int64_t qo = is.qo, ko = is.ko;
        const int Lq = is.Lq, Lk = is.Lk;
        const int q0 = qt * kBwdRows;
        const ColRange cr = visible_cols(Lq, Lk, q0, kBwdRows, causal, window, 0, bsh);
        const int kt_lo = cr.hi > cr.lo ? (int)(cr.lo / kBwdStage) : 0;
        const int kt_hi = cr.hi > cr.lo ? (int)((cr.hi + kBwdStage - 1) / kBwdStage) : 0;
        const int qw0 = q0 + 32 * wave;
        const int my_row = qw0 + col;
        const bool row_ok = my_row < Lq;
        const VisRange vis = keys_seen_by(my_row, Lk, causal, window, bsh);
        const int64_t qrow = (qo + my_row) * rs + (int64_t)h * D + KP * grp;

        // Q^T and dO^T as B operands; for softmax Di from O and dO in the same
        // layout.
        frag qf[C::NS], dof[C::NS];
        float di = 0.0f;
        // The wave's quarter of the second stage buffer: free until this item's
        // first barrier, and again after its last.
        using RT = RowTurn<D>;
        char* const wreg = (wave < 2 ? lds_k1 : lds_v1) + (wave & 1) * RT::BYTES;
        if constexpr (KP == 8) {
            // Whole rows in (16 bytes per lane), fragments out of LDS.
            const int64_t wrow = (qo + qw0) * rs + (int64_t)h * D;
            bf16x8 rq[RT::N], rd[RT::N], ro[ACT == ACT_SOFTMAX ? RT::N : 1];
            RT::load(rq, (const bf16*)a.q + wrow, rs, Lq - qw0, lane);
            RT::load(rd, (const bf16*)a.dout + wrow, rs, Lq - qw0, lane);
            if constexpr (ACT == ACT_SOFTMAX) RT::load(ro, (const bf16*)a.out + wrow, rs, Lq - qw0, lane);
            RT::put(wreg, rq, lane);
            RT::frags(qf, wreg, lane);
            RT::put(wreg, rd, lane);
            RT::frags(dof, wreg, lane);
            if constexpr (ACT == ACT_SOFTMAX) {
                frag of[C::NS];
                RT::put(wreg, ro, lane);
                RT::frags(of, wreg, lane);
#pragma unroll
                for (int s = 0; s < C::NS; ++s)
#pragma unroll
                    for (int e = 0; e < 8; ++e) di = fmaf((float)dof[s][e], (float)of[s][e], di);
            }
        } else {
            const T* qs = (const T*)a.q + qrow;
            const T* ds = (const T*)a.dout + qrow;
            const T* os = (const T*)a.out + qrow;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                qf[s] = row_ok ? *(const frag*)(qs + 2 * KP * s) : Frag<T>::zero();
                dof[s] = row_ok ? *(const frag*)(ds + 2 * KP * s) : Frag<T>::zero();
                if constexpr (ACT == ACT_SOFTMAX) {
                    const frag of = row_ok ? *(const frag*)(os + 2 * KP * s) : Frag<T>::zero();
                    di = fmaf(dof[s], of, di);
                }
            }
        }
        float nlse2 = 0.0f;
        if constexpr (ACT == ACT_SOFTMAX) {
            di = halves_sum(di);
            nlse2 = row_ok ? -a.lse[(qo + my_row) * a.H + h] * kLog2e : 0.0f;
            if (row_ok && grp == 0) {
                a.di[(qo + my_row) * a.H + h] = di;
                a.nl2[(qo + my_row) * a.H + h] = nlse2;  // the dK/dV pass's exponent offsets
            }
        }
        const float inv_lk = Lk > 0 ? 1.0f / (float)Lk : 0.0f;

        floatx16 dqacc[C::ND];
#pragma unroll
        for (int i = 0; i < C::ND; ++i) dqacc[i] = floatx16{};

        const char* Kseq = (const char*)a.k + (ko * rs + (int64_t)h * D) * (int)sizeof(T);
        const char* Vseq = (const char*)a.v + (ko * rs + (int64_t)h * D) * (int)sizeof(T);
        auto issue = [&](int kt, char* kdst, char* vdst) {
            const int kbase = kt * kBwdStage;
            const uint32_t nrec =
                __builtin_amdgcn_readfirstlane((uint32_t)min(max(Lk - kbase, 0), kBwdStage) * rsb);
            ld.issue(Kseq + (int64_t)kbase * rsb, nrec, kdst, wave);
            ld.issue(Vseq + (int64_t)kbase * rsb, nrec, vdst, wave);
        };

        auto stage = [&](int kt, const char* kl, const char* vl, char* kn, char* vn) {
            if (!kSingleStage && kt + 1 < kt_hi) issue(kt + 1, kn, vn);
            const int kw0 = kt * kBwdStage;
            const bool skip = wave_skips(vis, row_ok, kw0, kBwdStage);
            if (!skip) {
                const bool need_mask = wave_needs_mask(vis, row_ok, kw0, kBwdStage);
                frag dsf[C::NB][C::NT];
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    floatx16 sacc = floatx16{}, dpacc = floatx16{};
                    const char* kblk = kl + nb * 32 * C::ROWB;
                    const char* vblk = vl + nb * 32 * C::ROWB;
                    // K and V rows read two k-steps ahead of their products (the
                    // scheduling barriers keep each read from sinking next to its
                    // product, which would expose the LDS latency per product).
                    frag kr[2], vr[2];
#pragma unroll
                    for (int s = 0; s < 2 && s < C::NS; ++s) {
                        kr[s] = C::STile::read_rows(kblk, koff[s]);
                        vr[s] = C::STile::read_rows(vblk, koff[s]);
                    }
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) {
                        __builtin_amdgcn_sched_barrier(0);
                        sacc = M::run(kr[s & 1], qf[s], sacc);
                        dpacc = M::run(vr[s & 1], dof[s], dpacc);
                        if (s + 2 < C::NS) {
                            kr[s & 1] = C::STile::read_rows(kblk, koff[s + 2]);
                            vr[s & 1] = C::STile::read_rows(vblk, koff[s + 2]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float g;
                        if constexpr (ACT == ACT_SOFTMAX) {
                            g = fast_exp2(fmaf(sacc[r], c_exp, nlse2)) * (dpacc[r] - di);
                        } else {
                            float act, dact;
                            pointwise_grad<ACT>(sacc[r] * a.scale, act, dact);
                            g = dact * dpacc[r] * inv_lk;
                        }
                        sacc[r] = g;
                    }
                    // One wave-uniform branch per block, not a select per element.
                    if (need_mask) {
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            sacc[r] = vis.has(kw0 + nb * 32 + key_of_reg<KP>(grp, r)) ? sacc[r] : 0.0f;
                    }
#pragma unroll
                    for (int t = 0; t < C::NT; ++t) dsf[nb][t] = to_frag<T>(sacc, KP * t);
                }
                // dQ^T += K^T dS^T: K^T fragments read three products ahead.
                constexpr int NQ = C::NB * C::NT * C::ND;
                auto ktr = [&](int i) __attribute__((always_inline)) {
                    return C::STile::read_tr(kl + (i / (C::NT * C::ND)) * 32 * C::ROWB, (i / C::ND) % C::NT, toff,
                                             i % C::ND);
                };
                frag ring[3];
#pragma unroll
                for (int i = 0; i < 3 && i < NQ; ++i) ring[i] = ktr(i);
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int db = i % C::ND;
                    dqacc[db] = M::run(ring[i % 3], dsf[i / (C::NT * C::ND)][(i / C::ND) % C::NT], dqacc[db]);
                    if (i + 3 < NQ) ring[i % 3] = ktr(i + 3);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
        };

        if constexpr (kSingleStage) {
            for (int kt = kt_lo; kt < kt_hi; ++kt) {
                issue(kt, lds_k0, lds_v0);
                __syncthreads();
                stage(kt, lds_k0, lds_v0, lds_k1, lds_v1);  // loads nothing, ends on a barrier
            }
        } else {
            if (kt_hi > kt_lo) {
                issue(kt_lo, lds_k0, lds_v0);
                __syncthreads();
            }
            for (int kt = kt_lo; kt < kt_hi; kt += 2) {
                stage(kt, lds_k0, lds_v0, lds_k1, lds_v1);
                if (kt + 1 < kt_hi) stage(kt + 1, lds_k1, lds_v1, lds_k0, lds_v0);
            }
        }

        if (tid == 0) pend = xq_issue(a.q_counters, s_xq);
        if constexpr (KP == 8 && sizeof(GT) == 2) {
            // Whole rows out through the wave's region (the stage loop ended on a
            // barrier, or loaded nothing).
            RT::put_acc(wreg, dqacc, a.scale, lane);
            RT::store((bf16*)a.dq + (qo + qw0) * rs + (int64_t)h * D, rs, Lq - qw0, wreg, lane);
        } else if (row_ok) {
            // fp32 gradients (or fp32 inputs): 16 bytes of one row per lane and store.
            GT* dst = (GT*)a.dq + (qo + my_row) * rs + (int64_t)h * D + 4 * grp;
            const float sc = a.scale;
#pragma unroll
            for (int i = 0; i < C::ND; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    store4<GT>(dst + 32 * i + 8 * j, dqacc[i][4 * j] * sc, dqacc[i][4 * j + 1] * sc,
                               dqacc[i][4 * j + 2] * sc, dqacc[i][4 * j + 3] * sc);
        }
    }
#else
    (void)a;
#endif
}

// dK/dV pass -------------------------------------------------------------------
// Occupancy the pass is compiled for (waves per SIMD, lowest and highest). d <= 64
// runs two workgroups per CU: pinning two waves lets the compiler keep both
// accumulator sets in ordinary registers (4 % faster on w4). d = 128 keeps the
// default range (it holds ~370 registers and runs one wave per SIMD).
template <int D> constexpr int kDkdvWavesMin = D == 128 ? 1 : 2;
template <int D> constexpr int kDkdvWavesMax = D == 128 ? 8 : 2;

template <typename T, int D, int ACT, typename GT>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(kDkdvWavesMin<D>, kDkdvWavesMax<D>))) void ja_bwd_dkdv_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = BwdCfg<T, D>;
    using M = Mma<T>;
    typedef typename Frag<T>::type frag;
    constexpr int KP = C::KP;

    __shared__ __attribute__((aligned(1024))) char lds_q0[C::STile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_o0[C::STile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_q1[C::STile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_o1[C::STile::BYTES];
    __shared__ __attribute__((aligned(256))) float lds_l0[kBwdStage];
    __shared__ __attribute__((aligned(256))) float lds_d0[kBwdStage];
    __shared__ __attribute__((aligned(256))) float lds_l1[kBwdStage];
    __shared__ __attribute__((aligned(256))) float lds_d1[kBwdStage];
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, grp = lane >> 5;
    const int total = a.k_counters[kCtrTotal];
    const int64_t rs = (int64_t)a.H * D;
    const uint32_t rsb = (uint32_t)(rs * (int)sizeof(T));
    const uint32_t hsb = (uint32_t)(a.H * 4);  // stride of one row of lse / Di, bytes
    const int causal = a.causal, window = a.window, bsh = a.bsh;
    const float c_exp = a.scale * kLog2e;

    int roff[C::NS];
    int toff[C::ND][2];
    C::STile::row_offsets(col, grp, roff);
    C::STile::tr_offsets(lane, toff);
    typename C::Loader ld;
    ld.init(wave, lane, rsb);

    __shared__ int s_xq[2];
    int pend = 0;  // thread 0's pop in flight, sent before the previous item's output
    if (tid == 0) {
        xq_init(s_xq, a.window > 0);
        pend = xq_issue(a.k_counters, s_xq);
    }
    for (;;) {
        __syncthreads();
        if (tid == 0) s_item = xq_resolve(a.k_counters, s_xq, pend, total);
        __syncthreads();
        const int idx = __builtin_amdgcn_readfirstlane(s_item);
        if (idx >= total) break;
        const int pair = idx / a.H, h = idx - pair * a.H;
        const ItemSeq is = load_item(a.k_items, pair, true, a.Tq, a.Tk);
        const int kt = is.t;
        const int64_t qo = is.qo, ko = is.ko;
        const int Lq = is.Lq, Lk = is.Lk;
        const int k0 = kt * kBwdRows;
        const ColRange cr = visible_cols(Lk, Lq, k0, kBwdRows, causal, window, 1, bsh);
        const int qs_lo = cr.hi > cr.lo ? (int)(cr.lo / kBwdStage) : 0;
        const int qs_hi = cr.hi > cr.lo ? (int)((cr.hi + kBwdStage - 1) / kBwdStage) : 0;
        // A tile of at most 64 keys (short K/V, or a sequence's last tile) would
        // leave two waves without keys: then, if it visits at least two query
        // stages (both pairs get work), waves w and w + 2 share keys [32 (w % 2),
        // +32) and split each stage's queries (wave pair p takes the stage's
        // 32-query block p); the pairs add their partial dK, dV at the end.
        const bool pair_split = Lk - k0 <= 64 && qs_hi - qs_lo >= 2;  // uniform over the workgroup
        const int kwave = pair_split ? (wave & 1) : wave;
        const int kw0 = k0 + 32 * kwave;
        const int my_key = kw0 + col;
        const bool key_ok = my_key < Lk;
        const VisRange vis = queries_seeing(my_key, Lq, Lk, causal, window, bsh);
        const int64_t krow = (ko + my_key) * rs + (int64_t)h * D + KP * grp;

        const float inv_lk = Lk > 0 ? 1.0f / (float)Lk : 0.0f;
        frag kf[C::NS], vf[C::NS];
        // The wave's quarter of the second stage buffer: free until this item's
        // first barrier, and again after its last.
        using RT = RowTurn<D>;
        char* const wreg = (wave < 2 ? lds_q1 : lds_o1) + (wave & 1) * RT::BYTES;
        if constexpr (KP == 8) {
            const int64_t wrow = (ko + kw0) * rs + (int64_t)h * D;
            bf16x8 rk[RT::N], rv[RT::N];
            RT::load(rk, (const bf16*)a.k + wrow, rs, Lk - kw0, lane);
            RT::load(rv, (const bf16*)a.v + wrow, rs, Lk - kw0, lane);
            RT::put(wreg, rk, lane);
            RT::frags(kf, wreg, lane);
            RT::put(wreg, rv, lane);
            RT::frags(vf, wreg, lane);
        } else {
            const T* ks = (const T*)a.k + krow;
            const T* vs = (const T*)a.v + krow;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                kf[s] = key_ok ? *(const frag*)(ks + 2 * KP * s) : Frag<T>::zero();
                vf[s] = key_ok ? *(const frag*)(vs + 2 * KP * s) : Frag<T>::zero();
            }
        }
        floatx16 dkacc[C::ND], dvacc[C::ND];
#pragma unroll
        for (int i = 0; i < C::ND; ++i) {
            dkacc[i] = floatx16{};
            dvacc[i] = floatx16{};
        }

        const char* Qseq = (const char*)a.q + (qo * rs + (int64_t)h * D) * (int)sizeof(T);
        const char* Oseq = (const char*)a.dout + (qo * rs + (int64_t)h * D) * (int)sizeof(T);
        const char* Lseq = (const char*)(a.nl2 + qo * a.H + h);
        const char* Dseq = (const char*)(a.di + qo * a.H + h);
        auto issue = [&](int qs, char* qdst, char* odst, float* ldst, float* ddst) {
            const int qbase = qs * kBwdStage;
            const int nvalid = min(max(Lq - qbase, 0), kBwdStage);
            const uint32_t nrec = __builtin_amdgcn_readfirstlane((uint32_t)nvalid * rsb);
            ld.issue(Qseq + (int64_t)qbase * rsb, nrec, qdst, wave);
            ld.issue(Oseq + (int64_t)qbase * rsb, nrec, odst, wave);
            // -lse log2(e) and Di of the stage's queries: one 64-lane dword load each.
            if (ACT == ACT_SOFTMAX && wave < 2) {
                const uint32_t nrec_s = __builtin_amdgcn_readfirstlane((uint32_t)nvalid * hsb);
                const char* src = (wave == 0 ? Lseq : Dseq) + (int64_t)qbase * hsb;
                const __amdgpu_buffer_rsrc_t r =
                    __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, (int)nrec_s, 0x00020000);
                lds_char* dst = (lds_char*)(wave == 0 ? ldst : ddst);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, (uint32_t)lane * hsb, 0, 0, 0);
            }
        };

        auto stage = [&](int qs, const char* ql, const char* ol, const float* ll, const float* dl, char* qn,
                         char* on, float* ln, float* dn) {
            if (!kSingleStage && qs + 1 < qs_hi) issue(qs + 1, qn, on, ln, dn);
            const int qbase = qs * kBwdStage;
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                if (pair_split && nb != (wave >> 1)) continue;  // the other pair's block
                const int qb0 = qbase + nb * 32;  // first query of this block
                // Wave-uniform: lanes past the sequence end still feed the shared
                // matrix operands (their K/V rows are zero and masked below).
                const bool skip = wave_skips(vis, key_ok, qb0, 32);
                if (skip) continue;
                const bool need_mask = wave_needs_mask(vis, key_ok, qb0, 32);
                const char* qblk = ql + nb * 32 * C::ROWB;
                const char* oblk = ol + nb * 32 * C::ROWB;
                // Operands are read from LDS ahead of the products that consume them
                // (the scheduling barriers keep the compiler from sinking each read
                // next to its product, which would expose the LDS latency per product):
                // Q and dO rows for S and dP first, then the transposed dO and Q blocks
                // for dV and dK while S, dP and the softmax terms are computed.
                frag rq[C::NS], ro[C::NS];
#pragma unroll
                for (int s = 0; s < C::NS; ++s) {
                    rq[s] = C::STile::read_rows(qblk, roff[s]);
                    ro[s] = C::STile::read_rows(oblk, roff[s]);
                }
                __builtin_amdgcn_sched_barrier(0);
                floatx16 sacc = floatx16{}, dpacc = floatx16{};
#pragma unroll
                for (int s = 0; s < C::NS; ++s) {
                    sacc = M::run(rq[s], kf[s], sacc);
                    dpacc = M::run(ro[s], vf[s], dpacc);
                }
                __builtin_amdgcn_sched_barrier(0);
                frag tv[C::NT][C::ND], tk[C::NT][C::ND];
#pragma unroll
                for (int t = 0; t < C::NT; ++t)
#pragma unroll
                    for (int db = 0; db < C::ND; ++db) {
                        tv[t][db] = C::STile::read_tr(oblk, t, toff, db);
                        tk[t][db] = C::STile::read_tr(qblk, t, toff, db);
                    }
                __builtin_amdgcn_sched_barrier(0);
                // Register r holds query qb0 + key_of_reg(grp, r): for bf16 two runs
                // of 8 consecutive queries, read as float4s from lse / Di.
                float lse_r[16], di_r[16];
#pragma unroll
                for (int r = 0; r < 16 && ACT == ACT_SOFTMAX; r += 4) {
                    const int ql_ = nb * 32 + key_of_reg<KP>(grp, r);
                    if constexpr (KP == 8) {
                        const floatx4 l4 = *(const floatx4*)(ll + ql_);
                        const floatx4 d4 = *(const floatx4*)(dl + ql_);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            lse_r[r + e] = l4[e];
                            di_r[r + e] = d4[e];
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int qe = nb * 32 + key_of_reg<KP>(grp, r + e);
                            lse_r[r + e] = ll[qe];
                            di_r[r + e] = dl[qe];
                        }
                    }
                }
                floatx16 dsacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p, g;
                    if constexpr (ACT == ACT_SOFTMAX) {
                        p = fast_exp2(fmaf(sacc[r], c_exp, lse_r[r]));
                        g = p * (dpacc[r] - di_r[r]);
                    } else {
                        float act, dact;
                        pointwise_grad<ACT>(sacc[r] * a.scale, act, dact);
                        p = act * inv_lk;
                        g = dact * dpacc[r] * inv_lk;
                    }
                    sacc[r] = p;
                    dsacc[r] = g;
                }
                // One wave-uniform branch per block, not a select per element.
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const bool ok = vis.has(qb0 + key_of_reg<KP>(grp, r));
                        sacc[r] = ok ? sacc[r] : 0.0f;
                        dsacc[r] = ok ? dsacc[r] : 0.0f;
                    }
                }
#pragma unroll
                for (int t = 0; t < C::NT; ++t) {
                    const frag pf = to_frag<T>(sacc, KP * t);
                    const frag dsf = to_frag<T>(dsacc, KP * t);
#pragma unroll
                    for (int db = 0; db < C::ND; ++db) {
                        dvacc[db] = M::run(tv[t][db], pf, dvacc[db]);
                        dkacc[db] = M::run(tk[t][db], dsf, dkacc[db]);
                    }
                }
            }
            __syncthreads();
        };

        if constexpr (kSingleStage) {
            for (int qs = qs_lo; qs < qs_hi; ++qs) {
                issue(qs, lds_q0, lds_o0, lds_l0, lds_d0);
                __syncthreads();
                stage(qs, lds_q0, lds_o0, lds_l0, lds_d0, lds_q1, lds_o1, lds_l1, lds_d1);  // ends on a barrier
            }
        } else {
            if (qs_hi > qs_lo) {
                issue(qs_lo, lds_q0, lds_o0, lds_l0, lds_d0);
                __syncthreads();
            }
            for (int qs = qs_lo; qs < qs_hi; qs += 2) {
                stage(qs, lds_q0, lds_o0, lds_l0, lds_d0, lds_q1, lds_o1, lds_l1, lds_d1);
                if (qs + 1 < qs_hi) stage(qs + 1, lds_q1, lds_o1, lds_l1, lds_d1, lds_q0, lds_o0, lds_l0, lds_d0);
            }
        }

        if (pair_split) {
            // Waves 2 and 3 hand their partial sums to waves 0 and 1 through the
            // stage buffers (free: the stage loop ended on a barrier, or loaded
            // nothing); each array holds one accumulator set of one wave.
            static_assert(C::ND * 16 * 64 * 4 <= C::STile::BYTES, "partial sums must fit a stage array");
            float* pk = (float*)((wave & 1) ? lds_q1 : lds_q0);
            float* pv = (float*)((wave & 1) ? lds_o1 : lds_o0);
            if (wave >= 2) {
#pragma unroll
                for (int i = 0; i < C::ND; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        pk[(i * 16 + r) * 64 + lane] = dkacc[i][r];
                        pv[(i * 16 + r) * 64 + lane] = dvacc[i][r];
                    }
            }
            __syncthreads();
            if (wave < 2) {
#pragma unroll
                for (int i = 0; i < C::ND; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        dkacc[i][r] += pk[(i * 16 + r) * 64 + lane];
                        dvacc[i][r] += pv[(i * 16 + r) * 64 + lane];
                    }
            }
            __syncthreads();  // the partial sums are read before the row turnarounds reuse the buffers
        }
        if (tid == 0) pend = xq_issue(a.k_counters, s_xq);
        const bool owner = !pair_split || wave < 2;  // writes its keys' dK, dV
        if (!owner) {
        } else if constexpr (KP == 8 && sizeof(GT) == 2) {
            // Whole rows out through the wave's region (the stage loop ended on a
            // barrier, or loaded nothing): dK, then dV.
            const int64_t wrow = (ko + kw0) * rs + (int64_t)h * D;
            RT::put_acc(wreg, dkacc, a.scale, lane);
            RT::store((bf16*)a.dk + wrow, rs, Lk - kw0, wreg, lane);
            RT::put_acc(wreg, dvacc, 1.0f, lane);
            RT::store((bf16*)a.dv + wrow, rs, Lk - kw0, wreg, lane);
        } else if (key_ok) {
            // fp32 gradients (or fp32 inputs): 16 bytes of one row per lane and store.
            const int64_t base = (ko + my_key) * rs + (int64_t)h * D + 4 * grp;
            GT* dk = (GT*)a.dk + base;
            GT* dv = (GT*)a.dv + base;
            const float sc = a.scale;
#pragma unroll
            for (int i = 0; i < C::ND; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    store4<GT>(dk + 32 * i + 8 * j, dkacc[i][4 * j] * sc, dkacc[i][4 * j + 1] * sc,
                               dkacc[i][4 * j + 2] * sc, dkacc[i][4 * j + 3] * sc);
                    store4<GT>(dv + 32 * i + 8 * j, dvacc[i][4 * j], dvacc[i][4 * j + 1], dvacc[i][4 * j + 2],
                               dvacc[i][4 * j + 3]);
                }
        }
    }
#else
    (void)a;
#endif
}

// dK/dV pass, role-split form (d = 128) --------------------------------------------
// Eight waves per workgroup, one workgroup per CU, two waves per SIMD: waves w and
// w + 4 (one SIMD) own the same 32 keys of the 128-key item. Wave w (the P wave)
// holds K as the B operand and forms S = Q K^T, the weights P (softmax: exp(S -
// lse); SiLU / GELU: act(Z) / Lk) and dV^T += dO^T P; wave w + 4 (the dS wave) holds
// V and forms dP = dO V^T, dS and dK^T += Q^T dS. Per 64-query stage the P wave
// hands its per-score factor for dS (softmax: P; SiLU / GELU: act'(Z) / Lk, zero
// where masked) to its partner through LDS, between the two halves of the stage.
// Each wave keeps one accumulator set and one operand set, so both fit the
// registers of two waves per SIMD, and one wave's vector work (the exponentials,
// dS) overlaps its partner's matrix products. Every product is formed as in
// ja_bwd_dkdv_kernel, in the same order.
constexpr int kKv2Waves = 8;
constexpr int kKv2Threads = 64 * kKv2Waves;
// Tag that selects the role-split form of the dK/dV kernel (same kernel name in traces).
struct RolePair {};

template <typename T, int D, int ACT, typename GT>
__global__ __launch_bounds__(kKv2Threads, 1) void ja_bwd_dkdv_kernel(BwdArgs a, RolePair) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = BwdCfg<T, D>;
    using M = Mma<T>;
    typedef typename Frag<T>::type frag;
    constexpr int KP = C::KP;
    static_assert(KP == 8 && C::NB == 2 && C::NT == 2, "bf16, 64-query stages");
    using Loader = TileLoader<typename C::STile, kKv2Waves>;

    __shared__ __attribute__((aligned(1024))) char lds_q0[C::STile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_o0[C::STile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_q1[C::STile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_o1[C::STile::BYTES];
    __shared__ __attribute__((aligned(256))) float lds_l0[kBwdStage];
    __shared__ __attribute__((aligned(256))) float lds_d0[kBwdStage];
    __shared__ __attribute__((aligned(256))) float lds_l1[kBwdStage];
    __shared__ __attribute__((aligned(256))) float lds_d1[kBwdStage];
    // Hand-over of the dS factor: [key block][query block][register quad][lane].
    __shared__ __attribute__((aligned(256))) floatx4 xch[4][C::NB][4][64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool pw = wave < 4;  // the P wave of its pair (else the dS wave)
    const int kb = wave & 3;   // the pair's 32-key block
    const int col = lane & 31, grp = lane >> 5;
    const int total = a.k_counters[kCtrTotal];
    const int64_t rs = (int64_t)a.H * D;
    const uint32_t rsb = (uint32_t)(rs * (int)sizeof(T));
    const uint32_t hsb = (uint32_t)(a.H * 4);
    const int causal = a.causal, window = a.window, bsh = a.bsh;
    const float c_exp = a.scale * kLog2e;

    int toff[C::ND][2];
    const int rx = C::STile::row_offset_base(col, grp);  // one register for the row-operand offsets
    C::STile::tr_offsets(lane, toff);
    Loader ld;
    ld.init(wave, lane, rsb);

    // One work item: a (sequence, head, 128-key tile) and the query stages its keys see.
    struct Item {
        int h, Lq, Lk, k0, qs_lo, qs_hi;
        int qo, ko;  // first query / key row of the sequence (row indices fit 32 bits)
    };
    auto geometry = [&](int idx, const ItemSeq& is) {
        Item it;
        it.h = idx - (idx / a.H) * a.H;
        it.qo = (int)is.qo;
        it.ko = (int)is.ko;
        it.Lq = is.Lq;
        it.Lk = is.Lk;
        it.k0 = is.t * kBwdRows;
        const ColRange cr = visible_cols(it.Lk, it.Lq, it.k0, kBwdRows, causal, window, 1, bsh);
        it.qs_lo = cr.hi > cr.lo ? (int)(cr.lo / kBwdStage) : 0;
        it.qs_hi = cr.hi > cr.lo ? (int)((cr.hi + kBwdStage - 1) / kBwdStage) : 0;
        return it;
    };
    // Query stage qs of an item (Q, dO rows; -lse log2(e), Di for softmax) into one set of stage arrays.
    auto issue = [&](const Item& it, int qs, char* qdst, char* odst, float* ldst, float* ddst) {
        const int qbase = qs * kBwdStage;
        const int nvalid = min(max(it.Lq - qbase, 0), kBwdStage);
        const uint32_t nrec = __builtin_amdgcn_readfirstlane((uint32_t)nvalid * rsb);
        const int64_t row0 = (int64_t)(it.qo + qbase) * rs + (int64_t)it.h * D;
        ld.issue((const char*)a.q + row0 * (int)sizeof(T), nrec, qdst, wave);
        ld.issue((const char*)a.dout + row0 * (int)sizeof(T), nrec, odst, wave);
        if (ACT == ACT_SOFTMAX && wave < 2) {
            const uint32_t nrec_s = __builtin_amdgcn_readfirstlane((uint32_t)nvalid * hsb);
            const float* src = (wave == 0 ? a.nl2 : a.di) + (int64_t)(it.qo + qbase) * a.H + it.h;
            const __amdgpu_buffer_rsrc_t r =
                __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, (int)nrec_s, 0x00020000);
            lds_char* dst = (lds_char*)(wave == 0 ? ldst : ddst);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, (uint32_t)lane * hsb, 0, 0, 0);
        }
    };
    // The wave's B operand: K rows (P wave) or V rows (dS wave) of its 32 keys.
    frag bf[C::NS];
    auto load_bf = [&](const Item& it, int ln) __attribute__((always_inline)) {
        const int key = it.k0 + 32 * kb + (ln & 31);
        const bool ok = key < it.Lk;
        const T* src = (const T*)(pw ? a.k : a.v) + (int64_t)(it.ko + key) * rs + (int64_t)it.h * D + KP * (ln >> 5);
#pragma unroll
        for (int s = 0; s < C::NS; ++s) bf[s] = ok ? *(const frag*)(src + 2 * KP * s) : Frag<T>::zero();
    };
    // (Double-buffered) an item's first query stage, into the first set of stage arrays.
    auto first_stage = [&](const Item& it) __attribute__((always_inline)) {
        if (!kSingleStage && it.qs_hi > it.qs_lo) issue(it, it.qs_lo, lds_q0, lds_o0, lds_l0, lds_d0);
    };
    // Four consecutive fp32 values of -lse log2(e) (or Di) for register run r of block nb.
    auto run4 = [&](const float* base, int nb, int r) __attribute__((always_inline)) {
        return *(const floatx4*)(base + nb * 32 + key_of_reg<KP>(grp, r));
    };

    // Items are popped one ahead and the next item's record is copied into LDS while
    // the current item runs, so that after its last stage the next item's K / V rows
    // and first query stage are requested before the current item's output is written
    // (their latency overlaps the output turnaround instead of following it).
    __shared__ int s_pop[2];
    __shared__ __attribute__((aligned(32))) int s_rec[kItemInts];
    __shared__ int s_xq[2];
    int pend = 0;  // thread 0's pop in flight
    if (tid == 0) {
        xq_init(s_xq, a.window > 0);
        s_pop[0] = xq_resolve(a.k_counters, s_xq, xq_issue(a.k_counters, s_xq), total);
        s_pop[1] = xq_resolve(a.k_counters, s_xq, xq_issue(a.k_counters, s_xq), total);
    }
    __syncthreads();
    int cur_idx = __builtin_amdgcn_readfirstlane(s_pop[0]);
    int nxt_idx = __builtin_amdgcn_readfirstlane(s_pop[1]);
    Item cur{};
    if (cur_idx < total) {
        cur = geometry(cur_idx, load_item(a.k_items, cur_idx / a.H, true, a.Tq, a.Tk));
        load_bf(cur, lane);
        first_stage(cur);
    }

    for (int it_n = 0; cur_idx < total; ++it_n) {
        __syncthreads();  // the item's first stage and K / V rows are in
        const bool nx_ok = nxt_idx < total;
        if (wave == 0 && lane < kItemInts && nx_ok) {
            // The next item's record, straight into LDS. It lands before the first
            // stage's closing barrier, which waits for vector memory.
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(a.k_items + kItemInts * (int64_t)(nxt_idx / a.H)), (short)0, 4 * kItemInts, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_char*)s_rec, 4, (uint32_t)lane * 4, 0, 0, 0);
        }
        const int h = cur.h, Lq = cur.Lq, Lk = cur.Lk, qs_lo = cur.qs_lo, qs_hi = cur.qs_hi;
        const int64_t ko = cur.ko;  // widened for the output addresses
        const int kw0 = cur.k0 + 32 * kb;
        const int my_key = kw0 + col;
        const bool key_ok = my_key < Lk;
        const VisRange vis = queries_seeing(my_key, Lq, Lk, causal, window, bsh);
        const float inv_lk = Lk > 0 ? 1.0f / (float)Lk : 0.0f;

        floatx16 acc[C::ND];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
        for (int i = 0; i < C::ND; ++i) acc[i] = floatx16{};

        auto stage = [&](int qs, const char* ql, const char* ol, const float* ll, const float* dl, char* qn,
                         char* on, float* ln, float* dn) {
            if (!kSingleStage && qs + 1 < qs_hi) issue(cur, qs + 1, qn, on, ln, dn);
            const int qbase = qs * kBwdStage;
            bool active[C::NB], need_mask[C::NB];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                active[nb] = !wave_skips(vis, key_ok, qbase + nb * 32, 32);
                need_mask[nb] = wave_needs_mask(vis, key_ok, qbase + nb * 32, 32);
            }
            // Each role's body reads its LDS arrays directly (never through a pointer
            // chosen by role), so the compiler can tell the current stage's arrays from
            // the ones the next stage is loading into and does not wait for that load.
            //
            // The stage runs in three phases split by two barriers, the dS wave one
            // query block behind the P wave, so that each wave's vector work meets
            // matrix products of its partner:
            //   phase 1: P: S, weights, factor of block 0      dS: dP of blocks 0 and 1
            //   phase 2: P: S, weights, factor of block 1;     dS: dS, dK of block 0
            //            dV of block 0
            //   phase 3: P: dV of block 1                      dS: dS, dK of block 1
            // Only LDS operations are waited for at the two inner barriers: the next
            // stage's loads stay in flight through them.
            if (pw) {
                frag pf[C::NB][C::NT];
                // S = Q K^T for block nb, the weights (kept as P fragments) and the dS
                // factor handed to the partner.
                auto weights = [&](int nb) __attribute__((always_inline)) {
                    const int qb0 = qbase + nb * 32;
                    frag ra[C::NS];
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) ra[s] = C::STile::read_rows(ql + nb * 32 * C::ROWB, C::STile::row_offset(rx, s));
                    __builtin_amdgcn_sched_barrier(0);
                    floatx16 c = floatx16{};
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) c = M::run(ra[s], bf[s], c);
                    __builtin_amdgcn_sched_barrier(0);
                    floatx4 l4[4];
                    if constexpr (ACT == ACT_SOFTMAX) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) l4[j] = run4(ll, nb, 4 * j);
                    }
                    floatx16 x;  // the dS factor handed to the partner
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float p, f;
                        if constexpr (ACT == ACT_SOFTMAX) {
                            p = fast_exp2(fmaf(c[r], c_exp, l4[r >> 2][r & 3]));
                            f = p;
                        } else {
                            float av, dav;
                            pointwise_grad<ACT>(c[r] * a.scale, av, dav);
                            p = av * inv_lk;
                            f = dav * inv_lk;
                        }
                        c[r] = p;
                        x[r] = f;
                    }
                    if (need_mask[nb]) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const bool ok = vis.has(qb0 + key_of_reg<KP>(grp, r));
                            c[r] = ok ? c[r] : 0.0f;
                            x[r] = ok ? x[r] : 0.0f;
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        xch[kb][nb][j][lane] = floatx4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
#pragma unroll
                    for (int t = 0; t < C::NT; ++t) pf[nb][t] = to_frag<T>(c, KP * t);
                };
                // dV^T += dO^T P for block nb.
                auto dv = [&](int nb) __attribute__((always_inline)) {
                    frag tf[C::NT][C::ND];
#pragma unroll
                    for (int t = 0; t < C::NT; ++t)
#pragma unroll
                        for (int db = 0; db < C::ND; ++db)
                            tf[t][db] = C::STile::read_tr(ol + nb * 32 * C::ROWB, t, toff, db);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < C::NT; ++t)
#pragma unroll
                        for (int db = 0; db < C::ND; ++db) acc[db] = M::run(tf[t][db], pf[nb][t], acc[db]);
                    __builtin_amdgcn_sched_barrier(0);
                };
                if (active[0]) weights(0);
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                if (active[1]) weights(1);
                if (active[0]) dv(0);
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                if (active[1]) dv(1);
            } else {
                floatx16 dpacc[C::NB];
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    if (!active[nb]) continue;
                    frag ra[C::NS];
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) ra[s] = C::STile::read_rows(ol + nb * 32 * C::ROWB, C::STile::row_offset(rx, s));
                    __builtin_amdgcn_sched_barrier(0);
                    floatx16 c = floatx16{};
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) c = M::run(ra[s], bf[s], c);
                    __builtin_amdgcn_sched_barrier(0);
                    dpacc[nb] = c;
                }
                // dS = factor o (dP - Di) (softmax) or factor o dP, then dK^T += Q^T dS,
                // for block nb once its factor is in LDS.
                auto dk = [&](int nb) __attribute__((always_inline)) {
                    floatx4 xf[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) xf[j] = xch[kb][nb][j][lane];
                    floatx4 d4[4];
                    if constexpr (ACT == ACT_SOFTMAX) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) d4[j] = run4(dl, nb, 4 * j);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    floatx16 g;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        if constexpr (ACT == ACT_SOFTMAX)
                            g[r] = xf[r >> 2][r & 3] * (dpacc[nb][r] - d4[r >> 2][r & 3]);
                        else
                            g[r] = xf[r >> 2][r & 3] * dpacc[nb][r];
                    }
                    frag gf[C::NT];
#pragma unroll
                    for (int t = 0; t < C::NT; ++t) gf[t] = to_frag<T>(g, KP * t);
                    frag tf[C::NT][C::ND];
#pragma unroll
                    for (int t = 0; t < C::NT; ++t)
#pragma unroll
                        for (int db = 0; db < C::ND; ++db)
                            tf[t][db] = C::STile::read_tr(ql + nb * 32 * C::ROWB, t, toff, db);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < C::NT; ++t)
#pragma unroll
                        for (int db = 0; db < C::ND; ++db) acc[db] = M::run(tf[t][db], gf[t], acc[db]);
                    __builtin_amdgcn_sched_barrier(0);
                };
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                if (active[0]) dk(0);
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                if (active[1]) dk(1);
            }
            __syncthreads();
        };

        if constexpr (kSingleStage) {
            for (int qs = qs_lo; qs < qs_hi; ++qs) {
                issue(cur, qs, lds_q0, lds_o0, lds_l0, lds_d0);
                __syncthreads();
                stage(qs, lds_q0, lds_o0, lds_l0, lds_d0, lds_q1, lds_o1, lds_l1, lds_d1);
            }
        } else {
            for (int qs = qs_lo; qs < qs_hi; qs += 2) {
                stage(qs, lds_q0, lds_o0, lds_l0, lds_d0, lds_q1, lds_o1, lds_l1, lds_d1);
                if (qs + 1 < qs_hi) stage(qs + 1, lds_q1, lds_o1, lds_l1, lds_d1, lds_q0, lds_o0, lds_l0, lds_d0);
            }
        }
        if (qs_hi <= qs_lo) __syncthreads();  // no stage ran: the record has landed after this

        // The lane index as a value the compiler cannot see through: what the epilogue
        // derives from it is computed here, not kept in registers across the stages.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        // Every stage array is free (the last stage ended on a barrier). The next item's
        // K / V rows go out first, then its first query stage (into the first set of stage
        // arrays), then this item's output. (Loaded after the stage loads, the rows made
        // the compiler wait for those loads before it issued them.)
        Item nxt{};
        if (nx_ok) {
            // The record as wave-uniform scalars (LDS reads land in vector registers).
            int rec[kItemInts];
#pragma unroll
            for (int i = 0; i < kItemInts; ++i) rec[i] = __builtin_amdgcn_readfirstlane(s_rec[i]);
            nxt = geometry(nxt_idx, item_from_record(rec, true, a.Tq, a.Tk));
        }
        load_bf(nxt, ln);  // without a next item: zeros, no load
        if (nx_ok) first_stage(nxt);
        if (tid == 0) pend = xq_issue(a.k_counters, s_xq);  // the item after the next one (returns during the turnaround)

        // Whole rows out through a wave-private region of the second set of stage
        // arrays (P waves) or of the dS hand-over array (dS waves): dV from the P waves,
        // dK (times scale) from the dS waves.
        const float sc = pw ? 1.0f : a.scale;
        GT* const dst = (GT*)(pw ? a.dv : a.dk);
        if constexpr (sizeof(GT) == 2) {
            using RT = RowTurn<D>;
            static_assert(2 * RT::BYTES == C::STile::BYTES, "two regions per stage array");
            static_assert(4 * RT::BYTES == sizeof(xch), "four regions in the hand-over array");
            char* const wreg = pw ? (wave < 2 ? lds_q1 : lds_o1) + (wave & 1) * RT::BYTES
                                  : (char*)&xch[0][0][0][0] + (wave - 4) * RT::BYTES;
            RT::put_acc(wreg, acc, sc, ln);
            RT::store((bf16*)dst + (ko + kw0) * rs + (int64_t)h * D, rs, Lk - kw0, wreg, ln);
        } else {
            if (key_ok) {
                GT* d = dst + (ko + my_key) * rs + (int64_t)h * D + 4 * grp;
#pragma unroll
                for (int i = 0; i < C::ND; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        store4<GT>(d + 32 * i + 8 * j, acc[i][4 * j] * sc, acc[i][4 * j + 1] * sc,
                                   acc[i][4 * j + 2] * sc, acc[i][4 * j + 3] * sc);
            }
        }
        if (tid == 0) s_pop[it_n & 1] = xq_resolve(a.k_counters, s_xq, pend, total);
        // The turnaround regions are read back and the pop is in LDS before any wave
        // moves on (the next item's first barrier then waits for its loads).
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        cur_idx = nxt_idx;
        nxt_idx = __builtin_amdgcn_readfirstlane(s_pop[it_n & 1]);
        cur = nxt;
    }
#else
    (void)a;
#endif
}

template <int D, int ACT, typename GT>
hipError_t launch_g(const BwdArgs& a, int grid_q, int grid_k, hipStream_t s, hipEvent_t before, hipEvent_t mid,
                    hipEvent_t after) {
    if (before && hipEventRecord(before, s) != hipSuccess) return hipErrorUnknown;
    hipLaunchKernelGGL((ja_bwd_dq_kernel<bf16, D, ACT, GT>), dim3(grid_q), dim3(kBwdThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mid && hipEventRecord(mid, s) != hipSuccess) return hipErrorUnknown;
    void (*const plain)(BwdArgs) = &ja_bwd_dkdv_kernel<bf16, D, ACT, GT>;
    void (*const pairs)(BwdArgs, RolePair) = &ja_bwd_dkdv_kernel<bf16, 128, ACT, GT>;
    if (D == 128 && a.kv_roles)
        hipLaunchKernelGGL(pairs, dim3(grid_k), dim3(kKv2Threads), 0, s, a, RolePair{});
    else
        hipLaunchKernelGGL(plain, dim3(grid_k), dim3(kBwdThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (after && hipEventRecord(after, s) != hipSuccess) return hipErrorUnknown;
    return hipSuccess;
}

template <int D, int ACT>
hipError_t launch_d(const BwdArgs& a, int grid_q, int grid_k, hipStream_t s, hipEvent_t before, hipEvent_t mid,
                    hipEvent_t after) {
    return a.grad_f32 ? launch_g<D, ACT, float>(a, grid_q, grid_k, s, before, mid, after)
                      : launch_g<D, ACT, bf16>(a, grid_q, grid_k, s, before, mid, after);
}

template <int D, int ACT, typename GT>
int occupancy_g(bool dkdv, bool roles) {
    int n = 0;
    void (*const dq)(BwdArgs) = &ja_bwd_dq_kernel<bf16, D, ACT, GT>;
    void (*const plain)(BwdArgs) = &ja_bwd_dkdv_kernel<bf16, D, ACT, GT>;
    void (*const pairs)(BwdArgs, RolePair) = &ja_bwd_dkdv_kernel<bf16, 128, ACT, GT>;
    const void* fn = !dkdv                 ? reinterpret_cast<const void*>(dq)
                     : (D == 128 && roles) ? reinterpret_cast<const void*>(pairs)
                                           : reinterpret_cast<const void*>(plain);
    const int threads = (dkdv && D == 128 && roles) ? kKv2Threads : kBwdThreads;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0) != hipSuccess) n = 1;
    return n > 0 ? n : 1;
}

template <int D, int ACT>
int occupancy_d(bool dkdv, bool grad_f32, bool roles) {
    return grad_f32 ? occupancy_g<D, ACT, float>(dkdv, roles) : occupancy_g<D, ACT, bf16>(dkdv, roles);
}

}  // namespace

bool bwd_supported(int dtype, int d, int act) {
    return dtype == 1 && (d == 32 || d == 64 || d == 128) && act >= ACT_SOFTMAX && act <= ACT_GELU_TAYLOR;
}

int bwd_rows_per_item() { return kBwdRows; }
int bwd_cols_per_stage() { return kBwdStage; }

template <int ACT>
hipError_t launch_a(const BwdArgs& a, int d, int grid_q, int grid_k, hipStream_t stream, hipEvent_t before,
                    hipEvent_t mid, hipEvent_t after) {
    switch (d) {
        case 32: return launch_d<32, ACT>(a, grid_q, grid_k, stream, before, mid, after);
        case 64: return launch_d<64, ACT>(a, grid_q, grid_k, stream, before, mid, after);
        case 128: return launch_d<128, ACT>(a, grid_q, grid_k, stream, before, mid, after);
        default: return hipErrorInvalidValue;
    }
}

template <int ACT>
int occupancy_a(int d, bool dkdv, bool grad_f32, bool roles) {
    switch (d) {
        case 32: return occupancy_d<32, ACT>(dkdv, grad_f32, false);
        case 64: return occupancy_d<64, ACT>(dkdv, grad_f32, false);
        case 128: return occupancy_d<128, ACT>(dkdv, grad_f32, roles);
        default: return 1;
    }
}

hipError_t launch_bwd(const BwdArgs& a, int d, int act, int grid_q, int grid_k, hipStream_t stream,
                      hipEvent_t before, hipEvent_t mid, hipEvent_t after) {
    switch (act) {
        case ACT_SOFTMAX: return launch_a<ACT_SOFTMAX>(a, d, grid_q, grid_k, stream, before, mid, after);
        case ACT_SILU: return launch_a<ACT_SILU>(a, d, grid_q, grid_k, stream, before, mid, after);
        case ACT_GELU: return launch_a<ACT_GELU>(a, d, grid_q, grid_k, stream, before, mid, after);
        case ACT_GELU_TAYLOR: return launch_a<ACT_GELU_TAYLOR>(a, d, grid_q, grid_k, stream, before, mid, after);
        default: return hipErrorInvalidValue;
    }
}

int bwd_blocks_per_cu(int d, int act, bool dkdv, bool grad_f32, bool roles) {
    switch (act) {
        case ACT_SOFTMAX: return occupancy_a<ACT_SOFTMAX>(d, dkdv, grad_f32, roles);
        case ACT_SILU: return occupancy_a<ACT_SILU>(d, dkdv, grad_f32, roles);
        case ACT_GELU: return occupancy_a<ACT_GELU>(d, dkdv, grad_f32, roles);
        case ACT_GELU_TAYLOR: return occupancy_a<ACT_GELU_TAYLOR>(d, dkdv, grad_f32, roles);
        default: return 1;
    }
}

}  // namespace ja
