// ja_fwd.hip -- fused jagged attention forward for gfx950.
//
// Computes, per (sequence, head), out = act(scale Q K^T, masks) V on the jagged
// rows of that sequence only ("Jagged Sequence Flash Attention" and "Generalized
// Dot-Product Attention (GDPA)" sections of the GEM training post): act is an
// online softmax (running max, running sum, rescaled accumulator) or a pointwise
// SiLU / tanh-GELU normalised by 1/Lk with no max, no rescale and no correction
// stage. Key tiles that no query of a work item can see (causal diagonal, window
// edges: "BlockAttention" section) are never loaded.
//
// Work decomposition. A persistent grid pops (sequence, query-tile, head) items,
// longest first, from the list ja_sched.hip built on the device.
//   * Standard layout: 4 waves, a 128-row query tile; wave w owns rows
//     [32w, 32w+32) and all waves share each 64-key stage in LDS. Two such
//     workgroups run on each CU, independently.
//   * Split layout (short queries, e.g. pooled attention with 32 seeds): the item
//     is a 32-row query tile; the waves split each stage's keys and merge their
//     partial results through LDS at the end.
//
// Per wave and 32-key block the scores are computed transposed, S^T = K Q^T, on
// the 32x32x16 bf16 matrix cores: A = K rows from LDS, B = the wave's queries
// held in registers for the whole item. In the C layout each lane then owns one
// query column, so the softmax statistics are per-lane scalars and a row
// reduction is a 16-register loop plus one permlane32 swap between the half-waves.
// P^T is already in the B-operand layout of the second product O^T += V^T P^T.
// The V^T operand is read from V's natural [key][d] layout with the LDS transpose
// read (ds_read_tr16_b64: each 16-lane group gathers 4 keys x 16 dims), and keys
// are permuted inside each 32-key block (key_of_arow) so that one lane's 8 keys
// are 2 x 4 consecutive rows.
//
// Memory path. K and V stages stream from HBM straight into LDS with buffer loads
// (no staging registers). The buffer descriptor of a stage ends at the sequence's
// last key, so keys past the end read as zero (softmax masks them; for SiLU/GELU
// act(0) = 0 and V = 0, so they contribute nothing). 16-byte chunks are
// XOR-swizzled per row so that both the matrix-operand reads of K and the
// transpose reads of V hit distinct LDS banks. Stages are double-buffered: the
// next stage's loads are issued before the current stage is consumed.
//
// Masks are evaluated only on blocks that cross the sequence end, the causal
// diagonal or a window edge; fully invisible blocks are skipped per wave.
// Softmax rescaling is lazy: the running max is only raised when a block exceeds
// it by more than 2^8, which leaves the result unchanged in exact arithmetic.
#include <math.h>

#include <type_traits>

#include "ja_common.h"
#include "ja_internal.h"
#include "ja_lds.h"
#include "ja_tiles.h"

namespace ja {
namespace {

template <typename T, int D, bool SPLIT>
struct FwdCfg {
    static constexpr int NW = SPLIT ? (D == 128 ? 4 : 8) : 4;  // waves per workgroup
    static constexpr int THREADS = 64 * NW;
    // Standard layout: two independent workgroups share each CU (64 KB of LDS and
    // at most 256 VGPRs each), so one's barriers and idle waves do not hold the
    // other's matrix work.
    static constexpr int MIN_BLOCKS = SPLIT ? 1 : 2;
    static constexpr int WQ = SPLIT ? 1 : NW;                 // query slices
    static constexpr int WK = NW / WQ;                        // key slices
    static constexpr int NB = SPLIT ? 1 : 2;                  // 32-key blocks per wave per stage
    static constexpr int BM = 32 * WQ;                        // query rows per item
    static constexpr int KT = 32 * NB * WK;                   // keys per stage
    static constexpr int KP = Mma<T>::KPACK;
    static constexpr int NS = D / (2 * KP);                   // k-steps of S^T over d
    static constexpr int NT = 32 / (2 * KP);                  // k-steps of P V per 32-key block
    static constexpr int ND = D / 32;                         // 32-row blocks of O^T
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int ROWB = D * ESZ;                      // bytes per K/V row in LDS
    static constexpr int CPR = ROWB / 16;                     // 16-byte chunks per row
    static constexpr int TILE_BYTES = KT * ROWB;              // K or V of one stage
    static constexpr int INSTR = TILE_BYTES / 1024;           // 64-lane x 16-byte loads per tile
    using KVTile = Tile<T, D, KT>;
    using Loader = TileLoader<KVTile, NW>;
    static constexpr int SLICE = 64 * (D / 2 + 2);            // floats one wave hands over when merging
    static_assert(TILE_BYTES % 1024 == 0, "tile must be whole 64-lane loads");
    // Merge slots alternate between two free stage arrays.
    static_assert(!SPLIT || ((WK / 2 + 1) / 2) * SLICE * 4 <= TILE_BYTES, "merge slots must fit");
    static_assert(D % (2 * KP) == 0 && D % 32 == 0, "unsupported head dim");
};

// XQ: pop from XCD-local work queues (built only for the sliding-window case they help;
// a separate instantiation, so the other kernels keep their registers).
template <typename T, int D, int ACT, bool SPLIT, int CHUNK, bool XQ = false,
          int NTHREADS = FwdCfg<T, D, SPLIT>::THREADS, int MINB = FwdCfg<T, D, SPLIT>::MIN_BLOCKS>
__global__ __launch_bounds__(NTHREADS, MINB) void ja_fwd_kernel(FwdArgs a) {
    // The body uses gfx950-only types and builtins; the host pass only needs the
    // kernel's signature for its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    using C = FwdCfg<T, D, SPLIT>;
    using M = Mma<T>;
    typedef typename Frag<T>::type frag;
    constexpr int KP = C::KP;

    // Two K/V stage buffers as four distinct arrays: the loads of one stage and the
    // reads of the other then have provably disjoint targets, so the compiler does
    // not wait for the prefetch before reading the current stage.
    __shared__ __attribute__((aligned(1024))) char lds_k0[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v0[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_k1[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v1[C::TILE_BYTES];
    __shared__ int s_item;
    __shared__ float s_max[SPLIT ? C::WK * 64 : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform by construction
    const int wq = SPLIT ? 0 : wave;
    const int wk = SPLIT ? wave : 0;
    const int col = lane & 31, grp = lane >> 5;
    const int total = a.counters[kCtrTotal];
    const T* __restrict__ Qg = (const T*)a.q;
    const char* __restrict__ Kg = (const char*)a.k;
    const char* __restrict__ Vg = (const char*)a.v;
    T* __restrict__ Og = (T*)a.out;
    const int64_t rs = (int64_t)a.H * D;          // token row stride, elements
    const uint32_t rsb = (uint32_t)(rs * C::ESZ);  // ... bytes
    const int causal = a.causal, window = a.window, bsh = a.bsh;

    // Softmax works in the exp2 domain. With scale > 0 the row max is taken on raw
    // scores and folded into one FMA per element; otherwise scores are scaled first.
    const bool prescale = !(a.scale > 0.0f);
    const float c_exp = prescale ? 1.0f : a.scale * kLog2e;

    // Per-lane constant LDS offsets: K as the row operand of S^T, V through
    // transpose reads, and the chunks this lane loads.
    int koff[C::NS];
    int voff[C::ND][2];
    C::KVTile::row_offsets(col, grp, koff);
    C::KVTile::tr_offsets(lane, voff);
    typename C::Loader ld;
    ld.init(wave, lane, rsb);

    // The next item is popped before the current item's output stores, and the
    // barriers between items only publish LDS: the atomic's return does not queue
    // behind the stores, and the stores drain while the next item starts.
    // Invariant that makes an LDS-only wait enough here: no buffer-to-LDS stage load
    // is outstanding at an item boundary. Every stage an item loads is consumed
    // before that item's last stage barrier (a __syncthreads, which waits for all
    // vector memory operations), and the next item issues its first load after
    // these barriers. The single-stage race-check build (JA_SINGLE_STAGE) exercises
    // the same boundaries with a wait and a barrier around every load.
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    __shared__ int s_xq[2];
    int pend = 0;  // thread 0's pop in flight
    if (tid == 0) {
        if constexpr (XQ) xq_init(s_xq, true);
        pend = XQ ? xq_issue(a.counters, s_xq) : atomicAdd(&a.counters[kCtrPop], 1);
    }
    for (;;) {
        if (tid == 0) s_item = XQ ? xq_resolve(a.counters, s_xq, pend, total) : pend;
        lds_barrier();
        const int idx = __builtin_amdgcn_readfirstlane(s_item);  // same for every lane
        lds_barrier();  // s_item is read by every wave before it is rewritten
        if (idx >= total) break;
        const int pair = idx / a.H, h = idx - pair * a.H;
        const ItemSeq is = load_item(a.items, pair, false, a.Tq, a.Tk);
        const int64_t qo = is.qo, ko = is.ko;
        const int Lq = is.Lq, Lk = is.Lk;
        const char* Kseq = Kg + (ko * rs + (int64_t)h * D) * C::ESZ;
        const char* Vseq = Vg + (ko * rs + (int64_t)h * D) * C::ESZ;

        // Chunked layout (CHUNK > 1, short keys and values): the item is CHUNK
        // consecutive query tiles of one sequence and head, processed one after the
        // other. When every row of the chunk sees keys of one stage only, that stage
        // is loaded once and stays in LDS for all of them, and each tile's queries
        // are prefetched into registers while the previous tile computes, so the
        // item streams queries in and outputs out with no per-tile load latency or
        // barrier ("outer-loop pipelining" for short K/V, GDPA section).
        const int c0 = is.t * C::BM * CHUNK;  // first query row of the item
        const int nsub = CHUNK == 1 ? 1 : max(1, min(CHUNK, (Lq - c0 + C::BM - 1) / C::BM));
        bool resident = false;
        int rkt = 0;
        if constexpr (CHUNK > 1) {
            const ColRange ccr = visible_cols(Lq, Lk, c0, C::BM * CHUNK, causal, window, 0, bsh);
            rkt = ccr.hi > ccr.lo ? (int)(ccr.lo / C::KT) : 0;
            resident = ccr.hi > ccr.lo && (int)((ccr.hi + C::KT - 1) / C::KT) == rkt + 1;
        }

        // Queries of a tile's wave slice as the B operand of S^T = K Q^T.
        auto load_q = [&](int row, frag (&dst)[C::NS]) __attribute__((always_inline)) {
            const bool ok = row < Lq;
            const T* src = Qg + (qo + row) * rs + (int64_t)h * D + KP * grp;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) dst[s] = ok ? *(const frag*)(src + 2 * KP * s) : Frag<T>::zero();
        };
        // Chunked layout: a wave's 32 query rows are read whole (16 bytes per lane,
        // CPR lanes per row) into registers, one tile ahead, and turned into
        // B-operand fragments through the wave's quarter of the second stage buffer.
        using RT = RowTurn<D>;
        bf16x8 qraw[CHUNK > 1 ? RT::N : 1];
        auto load_raw = [&](int row0) __attribute__((always_inline)) {
            if constexpr (CHUNK > 1)
                RT::load(qraw, (const bf16*)Qg + (qo + row0) * rs + (int64_t)h * D, rs, Lq - row0, lane);
        };
        char* const wreg = (wave < 2 ? lds_k1 : lds_v1) + (wave & 1) * RT::BYTES;  // wave-private
        frag qf[C::NS];
        if constexpr (CHUNK > 1) load_raw(c0 + 32 * wq);
        else load_q(c0 + 32 * wq + col, qf);

        for (int sub = 0; sub < nsub; ++sub) {
            const int q0 = c0 + sub * C::BM;
            const ColRange cr = visible_cols(Lq, Lk, q0, C::BM, causal, window, 0, bsh);
            const int kt_lo = cr.hi > cr.lo ? (int)(cr.lo / C::KT) : 0;
            const int kt_hi = cr.hi > cr.lo ? (int)((cr.hi + C::KT - 1) / C::KT) : 0;
            const int qw0 = q0 + 32 * wq;  // first query row of this wave
            const int my_row = qw0 + col;
            const bool row_ok = my_row < Lq;
            const VisRange vis = keys_seen_by(my_row, Lk, causal, window, bsh);
            if constexpr (CHUNK > 1) {
                // The region is free: the previous tile's output turnaround finished in
                // this wave's own order, and no stage load targets it before the next
                // barrier.
                RT::put(wreg, qraw, lane);
                RT::frags(qf, wreg, lane);
                if (sub + 1 < nsub) load_raw(qw0 + C::BM);
            }

            floatx16 oacc[C::ND];
#pragma unroll
            for (int i = 0; i < C::ND; ++i) oacc[i] = floatx16{};
            float m_run = -INFINITY, l_run = 0.0f;

            // Stage kt -> (kdst, vdst): K and V rows [kt*KT, kt*KT + KT) of this
            // sequence and head; rows at or past Lk read as zero.
            auto issue = [&](int kt, char* kdst, char* vdst) {
                const int kbase = kt * C::KT;
                const uint32_t nrec =
                    __builtin_amdgcn_readfirstlane((uint32_t)min(max(Lk - kbase, 0), C::KT) * rsb);
                ld.issue(Kseq + (int64_t)kbase * rsb, nrec, kdst, wave);
                ld.issue(Vseq + (int64_t)kbase * rsb, nrec, vdst, wave);
            };

            // Consume the stage in (kl, vl) while the next one (if any) streams into
            // (kn, vn).
            auto compute = [&](int kt, const char* kl, const char* vl) {
                const int kw0 = kt * C::KT + wk * 32 * C::NB;  // first key of this wave's blocks
                const bool skip = wave_skips(vis, row_ok, kw0, 32 * C::NB);
                if (!skip) {
                    // S^T = K Q^T for the wave's blocks, the blocks' chains interleaved and
                    // each K fragment read three products ahead of its use (the scheduling
                    // barriers keep the reads from sinking next to their products, which
                    // would expose the LDS latency on every product).
                    floatx16 sacc[C::NB];
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb) sacc[nb] = floatx16{};
                    constexpr int NSI = C::NB * C::NS;
                    auto kread = [&](int i) __attribute__((always_inline)) {
                        return C::KVTile::read_rows(kl + (wk * C::NB + i % C::NB) * 32 * C::ROWB, koff[i / C::NB]);
                    };
                    frag kr[3];
#pragma unroll
                    for (int i = 0; i < 3 && i < NSI; ++i) kr[i] = kread(i);
#pragma unroll
                    for (int i = 0; i < NSI; ++i) {
                        __builtin_amdgcn_sched_barrier(0);
                        sacc[i % C::NB] = M::run(kr[i % 3], qf[i / C::NB], sacc[i % C::NB]);
                        if (i + 3 < NSI) kr[i % 3] = kread(i + 3);
                    }
                    __builtin_amdgcn_sched_barrier(0);

                    // V^T fragments of O^T += V^T P^T, read ahead: the first RV before the
                    // weights (whose vector work hides their LDS latency), each later one RV
                    // products before its use. Left to itself the compiler reads each
                    // fragment next to its product and waits for it every time.
                    constexpr int NPV = C::NB * C::NT * C::ND, RV = 4;
                    auto vread = [&](int i) __attribute__((always_inline)) {
                        const int nb = i / (C::NT * C::ND), t = (i / C::ND) % C::NT, db = i % C::ND;
                        return C::KVTile::read_tr(vl + (wk * C::NB + nb) * 32 * C::ROWB, t, voff, db);
                    };
                    frag vr[RV];
#pragma unroll
                    for (int i = 0; i < RV; ++i) vr[i] = vread(i);
                    __builtin_amdgcn_sched_barrier(0);

                    const bool need_mask = wave_needs_mask(vis, row_ok, kw0, 32 * C::NB);
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
                                for (int r = 0; r < 16; ++r) {
                                    const int key = kw0 + nb * 32 + key_of_reg<KP>(grp, r);
                                    sacc[nb][r] = vis.has(key) ? sacc[nb][r] : -INFINITY;
                                }
                        }
                        float mx = -INFINITY;
#pragma unroll
                        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
                        mx = halves_max(mx) * c_exp;
                        if (__any(mx > m_run + 8.0f)) {
                            const float m_new = fmaxf(m_run, mx);
                            const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_run - m_new);
                            l_run *= alpha;
#pragma unroll
                            for (int i = 0; i < C::ND; ++i) oacc[i] *= alpha;
                            m_run = m_new;
                        }
                        const float msub = m_run == -INFINITY ? 0.0f : m_run;
                        float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const float p = fast_exp2(fmaf(sacc[nb][r], c_exp, -msub));
                                lsum[r & 3] += p;
                                sacc[nb][r] = p;
                            }
                        l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
                    } else {
#pragma unroll
                        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                float p = pointwise<ACT>(sacc[nb][r] * a.scale);
                                if (need_mask) {
                                    const int key = kw0 + nb * 32 + key_of_reg<KP>(grp, r);
                                    p = vis.has(key) ? p : 0.0f;
                                }
                                sacc[nb][r] = p;
                            }
                    }

                    // P^T in the B-operand layout, then O^T += V^T P^T.
                    frag pf[C::NB][C::NT];
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                        for (int t = 0; t < C::NT; ++t) pf[nb][t] = to_frag<T>(sacc[nb], KP * t);
#pragma unroll
                    for (int i = 0; i < NPV; ++i) {
                        __builtin_amdgcn_sched_barrier(0);
                        const int nb = i / (C::NT * C::ND), t = (i / C::ND) % C::NT, db = i % C::ND;
                        oacc[db] = M::run(vr[i % RV], pf[nb][t], oacc[db]);
                        if (i + RV < NPV) vr[i % RV] = vread(i + RV);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            auto stage = [&](int kt, const char* kl, const char* vl, char* kn, char* vn) {
                if (kt + 1 < kt_hi) issue(kt + 1, kn, vn);
                compute(kt, kl, vl);
                __syncthreads();
            };

            if (CHUNK > 1 && resident) {
                // The chunk's one stage: loaded by the first tile, read by all. A tile
                // whose rows see no key (kt_hi == kt_lo) skips it.
                if (sub == 0) {
                    issue(rkt, lds_k0, lds_v0);
                    __syncthreads();
                }
                if (kt_hi > kt_lo) compute(rkt, lds_k0, lds_v0);
            } else {
                if constexpr (kSingleStage) {
                    for (int kt = kt_lo; kt < kt_hi; ++kt) {
                        issue(kt, lds_k0, lds_v0);
                        __syncthreads();
                        compute(kt, lds_k0, lds_v0);
                        __syncthreads();
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
            }

            if (sub == nsub - 1 && tid == 0) pend = XQ ? xq_issue(a.counters, s_xq) : atomicAdd(&a.counters[kCtrPop], 1);

            // Split layout: merge the key slices (the loop ended on a barrier, or no
            // stage was loaded, so the stage buffers are free). Softmax first agrees on
            // the row max, then partial sums and accumulators are added pairwise.
            if constexpr (SPLIT) {
                if (ACT == ACT_SOFTMAX) {
                    s_max[wave * 64 + lane] = m_run;
                    __syncthreads();
                    float mg = -INFINITY;
#pragma unroll
                    for (int w = 0; w < C::WK; ++w) mg = fmaxf(mg, s_max[w * 64 + lane]);
                    const float sc = m_run == -INFINITY ? 0.0f : fast_exp2(m_run - mg);
                    l_run *= sc;
#pragma unroll
                    for (int i = 0; i < C::ND; ++i) oacc[i] *= sc;
                    m_run = mg;
                }
                // slot j: [D/2 + 2][64] floats at (j/2) * SLICE of lds_k0 (j even) or lds_v0 (j odd)
                auto slot = [&](int j) { return (float*)((j & 1) ? lds_v0 : lds_k0) + (j >> 1) * C::SLICE; };
#pragma unroll
                for (int half = C::WK / 2; half >= 1; half /= 2) {
                    if (wave >= half && wave < 2 * half) {
                        float* dst = slot(wave - half);
#pragma unroll
                        for (int i = 0; i < C::ND; ++i)
#pragma unroll
                            for (int r = 0; r < 16; ++r) dst[(i * 16 + r) * 64 + lane] = oacc[i][r];
                        dst[(D / 2) * 64 + lane] = l_run;
                    }
                    __syncthreads();
                    if (wave < half) {
                        const float* src = slot(wave);
#pragma unroll
                        for (int i = 0; i < C::ND; ++i)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[i][r] += src[(i * 16 + r) * 64 + lane];
                        l_run += src[(D / 2) * 64 + lane];
                    }
                    __syncthreads();
                }
            }

            if (!SPLIT || wave == 0) {
                float inv;
                float lse_val = 0.0f;
                if (ACT == ACT_SOFTMAX) {
                    const float l_tot = halves_sum(l_run);
                    inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
                    lse_val = l_tot > 0.0f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
                } else {
                    inv = Lk > 0 ? 1.0f / (float)Lk : 0.0f;
                }
                bool staged = false;
                if constexpr (!SPLIT && KP == 8) {
                    // The second stage buffer is free here (the stage loop ended on a
                    // barrier, resident chunks never load it): each wave turns its 32
                    // output rows around in its own quarter of it (16-byte chunks
                    // XOR-swizzled by row) and writes whole rows, 16 bytes per lane,
                    // instead of 8-byte pieces of 32 rows per instruction.
                    staged = true;
                    RT::put_acc(wreg, oacc, inv, lane);
                    RT::store((bf16*)Og + (qo + qw0) * rs + (int64_t)h * D, rs, Lq - qw0, wreg, lane);
                }
                if (my_row < Lq) {
                    if (!staged) {
                        T* dst = Og + (qo + my_row) * rs + (int64_t)h * D + 4 * grp;
#pragma unroll
                        for (int i = 0; i < C::ND; ++i)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                store4<T>(dst + 32 * i + 8 * j, oacc[i][4 * j] * inv, oacc[i][4 * j + 1] * inv,
                                          oacc[i][4 * j + 2] * inv, oacc[i][4 * j + 3] * inv);
                    }
                    if (ACT == ACT_SOFTMAX && a.lse != nullptr && grp == 0)
                        a.lse[(qo + my_row) * a.H + h] = lse_val;
                }
            }
        }  // sub-tiles
    }
#else
    (void)a;
#endif
}

// Layouts: 0 standard, 1 split (short queries), 2 chunked (short keys and values).
constexpr int kChunk = 4;  // query tiles per item in the chunked layout
template <int LAYOUT> struct LayoutOf {
    static constexpr bool split = LAYOUT == 1;
    static constexpr int chunk = LAYOUT == 2 ? kChunk : 1;
};

template <typename T, int D, int ACT, int LAYOUT>
hipError_t launch_one(const FwdArgs& a, int grid, hipStream_t stream) {
    using L = LayoutOf<LAYOUT>;
    // XCD-local queues for bf16, d = 128, standard layout under a sliding window: the
    // list then orders most tiles by sequence and tile, so an XCD's consecutive tiles
    // share K / V stages in its L2 (under a plain causal mask the tiles of one cost come
    // from many sequences, and the single queue measured faster).
    constexpr bool kXqBuilt = std::is_same<T, bf16>::value && D == 128 && LAYOUT == 0;
    if (kXqBuilt && a.window > 0)
        hipLaunchKernelGGL((ja_fwd_kernel<T, D, ACT, L::split, L::chunk, kXqBuilt>), dim3(grid),
                           dim3(FwdCfg<T, D, L::split>::THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((ja_fwd_kernel<T, D, ACT, L::split, L::chunk>), dim3(grid),
                           dim3(FwdCfg<T, D, L::split>::THREADS), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D, int ACT, int LAYOUT>
int occupancy_one() {
    using L = LayoutOf<LAYOUT>;
    int n = 0;
    const void* fn = reinterpret_cast<const void*>(&ja_fwd_kernel<T, D, ACT, L::split, L::chunk>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, FwdCfg<T, D, L::split>::THREADS, 0) != hipSuccess)
        return 1;
    return n > 0 ? n : 1;
}

// Dispatch over (dtype, d, act, layout) to a callable template F<T, D, ACT, LAYOUT>.
// The split and chunked layouts exist for bf16 only.
template <template <typename, int, int, int> class F, typename R, typename... Args>
R dispatch(int dtype, int d, int act, int layout, R fail, Args... args) {
#define JA_ACTS(T, D, LY)                                                 \
    switch (act) {                                                        \
        case ACT_SOFTMAX: return F<T, D, ACT_SOFTMAX, LY>::call(args...); \
        case ACT_SILU: return F<T, D, ACT_SILU, LY>::call(args...);       \
        case ACT_GELU: return F<T, D, ACT_GELU, LY>::call(args...);       \
        case ACT_GELU_TAYLOR: return F<T, D, ACT_GELU_TAYLOR, LY>::call(args...); \
        default: return fail;                                             \
    }
#define JA_DIMS(T, LY)              \
    switch (d) {                    \
        case 32: JA_ACTS(T, 32, LY)   \
        case 64: JA_ACTS(T, 64, LY)   \
        case 128: JA_ACTS(T, 128, LY) \
        default: return fail;       \
    }
    if (dtype == 1) {
        if (layout == 1) { JA_DIMS(bf16, 1) }
        if (layout == 2) { JA_DIMS(bf16, 2) }
        JA_DIMS(bf16, 0)
    }
    if (dtype == 0) { JA_DIMS(float, 0) }
#undef JA_DIMS
#undef JA_ACTS
    return fail;
}

template <typename T, int D, int ACT, int LAYOUT>
struct LaunchF {
    static hipError_t call(const FwdArgs* a, int grid, hipStream_t s) { return launch_one<T, D, ACT, LAYOUT>(*a, grid, s); }
};
template <typename T, int D, int ACT, int LAYOUT>
struct OccF {
    static int call() { return occupancy_one<T, D, ACT, LAYOUT>(); }
};
template <typename T, int D, int ACT, int LAYOUT>
struct ShapeF {
    static FwdShape call() {
        using L = LayoutOf<LAYOUT>;
        return FwdShape{FwdCfg<T, D, L::split>::BM * L::chunk, FwdCfg<T, D, L::split>::KT};
    }
};

}  // namespace

bool fwd_supported(int dtype, int d, int act) {
    return (dtype == 0 || dtype == 1) && (d == 32 || d == 64 || d == 128) && act >= ACT_SOFTMAX && act <= ACT_GELU_TAYLOR;
}

FwdShape fwd_shape(int dtype, int d, int act, int layout) {
    return dispatch<ShapeF, FwdShape>(dtype, d, act, dtype == 1 ? layout : 0, FwdShape{0, 0});
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int d, int act, int layout, int grid, hipStream_t stream) {
    return dispatch<LaunchF, hipError_t>(dtype, d, act, dtype == 1 ? layout : 0, hipErrorInvalidValue, &a, grid,
                                         stream);
}

int fwd_blocks_per_cu(int dtype, int d, int act, int layout) {
    return dispatch<OccF, int>(dtype, d, act, dtype == 1 ? layout : 0, 1);
}

}  // namespace ja
