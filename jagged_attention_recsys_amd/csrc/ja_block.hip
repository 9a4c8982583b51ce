// ja_block.hip -- fused backward of block-diagonal self-attention, one 64-token
// problem at a time.
//
// "BlockAttention" section of the GEM training post: with fixed token blocks each
// query block attends only to the keys and values of its own block, so the
// attention splits into independent small problems and the FlashAttention
// machinery that long rows need goes away: a row's keys all fit in one tile, so
// its softmax is recomputed exactly from that tile (no log-sum-exp from the
// forward) and Di comes from the same registers (no separate Di pass). This
// kernel handles blocks of up to 64 tokens: a workgroup of two waves solves one
// (64-token tile, head) problem at a time, wave w owning rows [32w, 32w + 32) of
// the tile, and walks the problems persistently (g, g + grid, ...). Blocks
// smaller than the tile are masked inside it. (The forward of such blocks runs
// the general forward kernel under the block mask: every row's keys then lie in
// one 64-key stage, so its online softmax takes a single step.)
//
// No atomics; each gradient row is written once. Q, K, V and dO of the tile
// stream into LDS. Query-stationary phase (each lane owns one query column, as
// in the general kernels): S^T = K Q^T and dP^T = V dO^T on the 32x32x16 bf16
// matrix cores, the row softmax over both 32-key blocks in one pass, then
// Di = sum_j P_ij dP_ij (which equals rowsum(dO o O)) and dS = P o (dP - Di);
// dQ^T = K^T dS^T from the registers. P and dS go to LDS as bf16 [query][key]
// tiles (over the V tile once V is consumed). Key-stationary phase: wave w takes
// keys [32w, 32w + 32) and forms dV^T = dO^T P and dK^T = Q^T dS with both
// operands read by LDS transpose reads.
#include <math.h>

#include "ja_block.h"
#include "ja_common.h"
#include "ja_internal.h"
#include "ja_lds.h"
#include "ja_tiles.h"

namespace ja {
namespace {

constexpr int kBlkWaves = 2;
constexpr int kBlkThreads = 64 * kBlkWaves;

template <int D>
struct BlkCfg {
    using RTile = Tile<bf16, D, kBlkTile>;           // Q, K, V or dO rows of one tile
    using PTile = Tile<bf16, kBlkTile, kBlkTile>;    // P or dS: [query][key], 64 x 64
    using Loader = TileLoader<RTile, kBlkWaves>;
    static constexpr int KP = 8;
    static constexpr int NS = RTile::NS;             // k-steps over d
    static constexpr int ND = RTile::ND;             // 32-row blocks of d
    static constexpr int NT = 32 / (2 * KP);         // k-steps per 32-key block
    static constexpr int ROWB = RTile::ROWB;
    // P and dS (8 KB each) overwrite the consumed V tile when it is large enough.
    static constexpr bool PS_IN_V = RTile::BYTES >= 2 * PTile::BYTES;
};

// B-operand offsets (queries as columns) of lane (col, grp) for rows 32w + col of
// a row tile, per k-step over d: the rows are not permuted.
template <int D>
__device__ __forceinline__ void bop_offsets(int row, int grp, int (&off)[BlkCfg<D>::NS]) {
    using RT = typename BlkCfg<D>::RTile;
#pragma unroll
    for (int s = 0; s < RT::NS; ++s) {
        const int c = 2 * s + grp;
        off[s] = row * RT::ROWB + ((c ^ swz<RT::CPR, 2>(row)) << 4);
    }
}

#if defined(__HIP_DEVICE_COMPILE__)
// Mask, then the one-pass row softmax of the two 32-key blocks of S^T (a lane's
// column is one query). Leaves exp2-domain p in s and returns the row sum; m2 is
// the exp2-domain max subtracted.
__device__ __forceinline__ float tile_softmax(floatx16 (&s)[2], bool nb1, bool need_mask, const VisRange& vis,
                                              int k0, int grp, float scale, float& m2) {
    const bool prescale = !(scale > 0.0f);
    const float c_exp = prescale ? 1.0f : scale * kLog2e;
    // Wave-uniform branches around whole loops, not selects per score.
    if (prescale) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[nb][r] *= scale * kLog2e;
    }
    if (need_mask) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[nb][r] = vis.has(k0 + nb * 32 + key_of_reg<8>(grp, r)) ? s[nb][r] : -INFINITY;
    }
    if (!nb1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[1][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
    mx = halves_max(mx) * c_exp;
    m2 = mx == -INFINITY ? 0.0f : mx;
    float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[nb][r], c_exp, -m2));
            lsum[r & 3] += p;
            s[nb][r] = p;
        }
    return halves_sum((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
}

// Workgroup barrier that publishes LDS only: outstanding global loads and
// stores are not waited for.
// Waits for LDS operations only: at the item boundaries where it is used no global
// load into LDS is outstanding (each tile's loads are waited for before the tile
// is read, with a wait on vector memory operations).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct TileItem {
    int h, L, r0, n;  // head, sequence length, first token of the tile, tokens in it
    int64_t o0;       // first row of the sequence
};

__device__ __forceinline__ bool tile_item(const BlkArgs& a, int idx, TileItem& it) {
    if (idx >= a.cap) return false;
    const int pair = idx / a.H;
    it.h = idx - pair * a.H;
    // Within the capacity the item is read before the count is known (one
    // dependent load fewer); entries past the count are stale and rejected.
    const int total = a.counters[kCtrTotal];
    typedef int int4v __attribute__((ext_vector_type(4)));
    const int4v rec = *(const int4v*)(a.items + kItemInts * (int64_t)pair);  // b, t, off[b], off[b+1]
    const int b = rec[0], t = rec[1];
    if (idx >= total || b < 0 || b >= a.B) return false;
    const int o0 = rec[2], o1 = rec[3];
    it.o0 = o0;
    // Rows are clamped to the tensors, so inconsistent offsets cannot reach
    // outside them.
    it.L = o0 < 0 ? 0 : min(o1, a.T) - o0;
    it.r0 = t * kBlkTile;
    it.n = min(it.L - it.r0, kBlkTile);
    return it.n > 0;
}
#endif

template <int D>
__global__ __launch_bounds__(kBlkThreads) void ja_blk_bwd_kernel(BlkArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = BlkCfg<D>;
    using M = Mma<bf16>;
    typedef bf16x8 frag;
    constexpr int KP = C::KP;

    __shared__ __attribute__((aligned(1024))) char lds_q[C::RTile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_k[C::RTile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v[C::RTile::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_o[C::RTile::BYTES];  // dO
    __shared__ __attribute__((aligned(1024))) char lds_ps[C::PS_IN_V ? 16 : 2 * C::PTile::BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, grp = lane >> 5;
    const int64_t rs = (int64_t)a.H * D;
    const uint32_t rsb = (uint32_t)(rs * 2);
    typename C::Loader ld;
    ld.init(wave, lane, rsb);
    const int qloc = 32 * wave + col;  // this lane's query (and key) row in the tile
    int koff[C::NS], boff[C::NS];
    int toff[C::ND][2], poff[2][2];
    C::RTile::row_offsets(col, grp, koff);
    bop_offsets<D>(qloc, grp, boff);
    C::RTile::tr_offsets(lane, toff);
    C::PTile::tr_offsets(lane, poff);

    // Persistent: workgroup g takes items g, g + grid, g + 2 grid, ...
    for (int idx = blockIdx.x;; idx += gridDim.x) {
    TileItem it;
    if (!tile_item(a, idx, it)) break;  // uniform over the workgroup
    const int64_t tile0 = (it.o0 + it.r0) * rs + (int64_t)it.h * D;
    lds_barrier();  // every wave is done with the previous item's LDS tiles
    const uint32_t nrec = __builtin_amdgcn_readfirstlane((uint32_t)it.n * rsb);
    ld.issue((const char*)a.k + tile0 * 2, nrec, lds_k, wave);
    ld.issue((const char*)a.v + tile0 * 2, nrec, lds_v, wave);
    ld.issue((const char*)a.q + tile0 * 2, nrec, lds_q, wave);
    ld.issue((const char*)a.dout + tile0 * 2, nrec, lds_o, wave);
    char* lds_p = C::PS_IN_V ? lds_v : lds_ps;
    char* lds_s = lds_p + C::PTile::BYTES;

    const int my_row = it.r0 + qloc;
    const bool row_ok = my_row < it.L;
    const VisRange vis = keys_seen_by(my_row, it.L, a.causal, 0, a.bsh);
    const bool nb1 = it.n > 32;
    const bool wave_rows = 32 * wave < it.n;  // this wave has query rows
    __syncthreads();

    // Query-stationary phase: S^T, dP^T, softmax, dS, dQ (kept in registers until
    // the end of the item).
    floatx16 sacc[2], dpacc[2];
    floatx16 dqacc[C::ND];
#pragma unroll
    for (int i = 0; i < C::ND; ++i) dqacc[i] = floatx16{};
    if (wave_rows) {
        frag qf[C::NS], dof[C::NS];
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            qf[s] = C::RTile::read_rows(lds_q, boff[s]);
            dof[s] = C::RTile::read_rows(lds_o, boff[s]);
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            sacc[nb] = floatx16{};
            dpacc[nb] = floatx16{};
            if (nb == 1 && !nb1) continue;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                sacc[nb] = M::run(C::RTile::read_rows(lds_k + nb * 32 * C::ROWB, koff[s]), qf[s], sacc[nb]);
                dpacc[nb] = M::run(C::RTile::read_rows(lds_v + nb * 32 * C::ROWB, koff[s]), dof[s], dpacc[nb]);
            }
        }
    }
    if (C::PS_IN_V) __syncthreads();  // every wave is done with V before P and dS overwrite it
    if (wave_rows) {
        const bool need_mask = wave_needs_mask(vis, row_ok, it.r0, kBlkTile);
        float m2;
        const float l = tile_softmax(sacc, nb1, need_mask, vis, it.r0, grp, a.scale, m2);
        const float inv = (l > 0.0f && row_ok) ? 1.0f / l : 0.0f;  // rows past the end: P = 0
        float di = 0.0f;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sacc[nb][r] *= inv;
                di = fmaf(sacc[nb][r], dpacc[nb][r], di);
            }
        di = halves_sum(di);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) dpacc[nb][r] = sacc[nb][r] * (dpacc[nb][r] - di);  // dS

        // P and dS rows to LDS ([query][key], this lane's row), 16 bytes per 8 keys.
        const int sw = swz<C::PTile::CPR, 2>(qloc);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c = 4 * nb + 2 * hh + grp;
                const int o = qloc * C::PTile::ROWB + ((c ^ sw) << 4);
                *(frag*)(lds_p + o) = to_frag<bf16>(sacc[nb], 8 * hh);
                *(frag*)(lds_s + o) = to_frag<bf16>(dpacc[nb], 8 * hh);
            }

        // dQ^T = K^T dS^T
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            if (nb == 1 && !nb1) continue;
#pragma unroll
            for (int t = 0; t < C::NT; ++t) {
                const frag dsf = to_frag<bf16>(dpacc[nb], KP * t);
#pragma unroll
                for (int db = 0; db < C::ND; ++db)
                    dqacc[db] = M::run(C::RTile::read_tr(lds_k + nb * 32 * C::ROWB, t, toff, db), dsf, dqacc[db]);
            }
        }
    } else {
        // No query rows: P and dS rows of this wave are zero.
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c = 4 * nb + 2 * hh + grp;
                const int o = qloc * C::PTile::ROWB + ((c ^ swz<C::PTile::CPR, 2>(qloc)) << 4);
                *(frag*)(lds_p + o) = frag{};
                *(frag*)(lds_s + o) = frag{};
            }
    }
    __syncthreads();

    // Key-stationary phase: wave w owns keys [32w, 32w + 32) of the tile (a wave
    // with no query rows has no keys either).
    floatx16 dkacc[C::ND], dvacc[C::ND];
#pragma unroll
    for (int i = 0; i < C::ND; ++i) {
        dkacc[i] = floatx16{};
        dvacc[i] = floatx16{};
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        if (nb == 1 && !nb1) continue;
        if (!wave_rows) continue;
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
            const frag pf = C::PTile::read_tr(lds_p + nb * 32 * C::PTile::ROWB, t, poff, wave);
            const frag sf = C::PTile::read_tr(lds_s + nb * 32 * C::PTile::ROWB, t, poff, wave);
#pragma unroll
            for (int db = 0; db < C::ND; ++db) {
                dvacc[db] = M::run(C::RTile::read_tr(lds_o + nb * 32 * C::ROWB, t, toff, db), pf, dvacc[db]);
                dkacc[db] = M::run(C::RTile::read_tr(lds_q + nb * 32 * C::ROWB, t, toff, db), sf, dkacc[db]);
            }
        }
    }
    // Every wave is done reading the tiles: each turns its 32 rows of dQ, dK and
    // dV around in its half of the K tile and writes whole rows (16 bytes per
    // lane) instead of 8-byte pieces of 32 rows per instruction.
    __syncthreads();
    if (wave_rows) {
        using RT = RowTurn<D>;
        char* const wreg = lds_k + wave * RT::BYTES;
        const int nrows = it.L - it.r0 - 32 * wave;
        const int64_t wrow = tile0 + (int64_t)(32 * wave) * rs;
        RT::put_acc(wreg, dqacc, a.scale, lane);
        RT::store((bf16*)a.dq + wrow, rs, nrows, wreg, lane);
        RT::put_acc(wreg, dkacc, a.scale, lane);
        RT::store((bf16*)a.dk + wrow, rs, nrows, wreg, lane);
        RT::put_acc(wreg, dvacc, 1.0f, lane);
        RT::store((bf16*)a.dv + wrow, rs, nrows, wreg, lane);
    }
    }
#else
    (void)a;
#endif
}

template <int D>
int blk_occupancy() {
    int n = 0;
    const void* fn = reinterpret_cast<const void*>(&ja_blk_bwd_kernel<D>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kBlkThreads, 0) != hipSuccess) n = 1;
    return n > 0 ? n : 1;
}

}  // namespace

bool blk_supported(int dtype, int d, int bsh) {
    return dtype == 1 && (d == 32 || d == 64 || d == 128) && bsh >= 0 && (1 << bsh) <= kBlkTile;
}

int blk_blocks_per_cu(int d) {
    switch (d) {
        case 32: return blk_occupancy<32>();
        case 64: return blk_occupancy<64>();
        case 128: return blk_occupancy<128>();
        default: return 1;
    }
}

hipError_t launch_blk_bwd(const BlkArgs& a, int d, int grid, hipStream_t s) {
    switch (d) {
        case 32: hipLaunchKernelGGL(ja_blk_bwd_kernel<32>, dim3(grid), dim3(kBlkThreads), 0, s, a); break;
        case 64: hipLaunchKernelGGL(ja_blk_bwd_kernel<64>, dim3(grid), dim3(kBlkThreads), 0, s, a); break;
        case 128: hipLaunchKernelGGL(ja_blk_bwd_kernel<128>, dim3(grid), dim3(kBlkThreads), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ja
