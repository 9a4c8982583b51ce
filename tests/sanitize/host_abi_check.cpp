// Host-side check of the C-ABI layer (ja_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, built with g++ for the CPU only (no GPU, no device
// code). The kernel launchers are replaced by stubs that launch nothing but check
// what the layer hands them: every workspace region the plan gives a launch
// (counters, per-sequence tile prefix, work lists, Di) must lie inside the
// caller's workspace, and the regions of one call must not overlap. main()
// calls every entry point over a sweep of sizes (empty, one, many and very long
// sequences, every head dim, dtype, activation and mask) with aligned fake device
// addresses that are never dereferenced, plus workspaces one byte short.
// Prints "ok" and exits 0 when every check holds; any sanitizer report aborts.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "jagged_attn.h"
#include "ja_block.h"
#include "ja_internal.h"
#include "ja_mx.h"

namespace {

uintptr_t g_ws_lo = 0, g_ws_hi = 0;  // the current call's workspace
struct Region {
    uintptr_t lo, hi;
};
std::vector<Region> g_regions;  // regions handed to launches of the current call
long g_launches = 0, g_failures = 0;

void fail(const char* what) {
    std::fprintf(stderr, "FAIL: %s\n", what);
    ++g_failures;
}

void region(const void* p, size_t bytes, const char* what) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p), hi = lo + bytes;
    if (lo < g_ws_lo || hi > g_ws_hi) fail(what);
    for (const Region& r : g_regions)
        if (lo < r.hi && r.lo < hi && !(lo == r.lo && hi == r.hi)) fail("workspace regions overlap");
    g_regions.push_back({lo, hi});
}

void begin_call(const void* ws, size_t bytes) {
    g_ws_lo = reinterpret_cast<uintptr_t>(ws);
    g_ws_hi = g_ws_lo + bytes;
    g_regions.clear();
}

}  // namespace

// --- stubs of the device side ----------------------------------------------------
namespace ja {

bool fwd_supported(int dtype, int d, int act) {
    return (dtype == 0 || dtype == 1) && (d == 32 || d == 64 || d == 128) && act >= 0 && act <= 3;
}
FwdShape fwd_shape(int dtype, int d, int act, int layout) {
    (void)act;
    if (dtype == 1 && layout == kLayoutSplit) return FwdShape{32, d == 128 ? 128 : 256};
    if (dtype == 1 && layout == kLayoutChunked) return FwdShape{512, 64};
    return FwdShape{128, 64};
}
int fwd_blocks_per_cu(int, int, int, int) { return 2; }
hipError_t launch_sched(const SchedArgs& a, hipStream_t) {
    ++g_launches;
    region(a.counters, sizeof(int32_t) * kCtrCount, "scheduler counters outside the workspace");
    region(a.tbase, sizeof(int32_t) * ((size_t)a.B + 1), "tile prefix outside the workspace");
    region(a.items, sizeof(int32_t) * kItemInts * (size_t)a.max_pairs, "work list outside the workspace");
    if (a.bm <= 0 || a.bn <= 0 || a.max_pairs < 0) fail("scheduler shape");
    return hipSuccess;
}
hipError_t launch_sched2(const SchedArgs& a, const SchedArgs& b, hipStream_t s) {
    --g_launches;  // one launch for both lists
    launch_sched(a, s);
    return launch_sched(b, s);
}
hipError_t launch_copy_items(const int32_t*, const int32_t*, int32_t*, int32_t*, int64_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_fwd(const FwdArgs& a, int, int, int, int, int grid, hipStream_t) {
    ++g_launches;
    if (grid < 1 || a.H < 1) fail("forward launch shape");
    return hipSuccess;
}
bool bwd_supported(int dtype, int d, int act) { return dtype == 1 && (d == 32 || d == 64 || d == 128) && act >= 0 && act <= 3; }
int bwd_rows_per_item() { return 128; }
int bwd_cols_per_stage() { return 64; }
hipError_t launch_bwd(const BwdArgs& a, int, int, int gq, int gk, hipStream_t, hipEvent_t, hipEvent_t, hipEvent_t) {
    ++g_launches;
    region(a.di, sizeof(float) * (size_t)a.Tq * (size_t)a.H, "Di outside the workspace");
    region(a.nl2, sizeof(float) * (size_t)a.Tq * (size_t)a.H, "exponent offsets outside the workspace");
    if (gq < 1 || gk < 1) fail("backward launch shape");
    return hipSuccess;
}
int bwd_blocks_per_cu(int, int, bool, bool, bool) { return 1; }
bool blk_supported(int dtype, int d, int bsh) { return dtype == 1 && (d == 32 || d == 64 || d == 128) && bsh <= 6; }
int blk_blocks_per_cu(int) { return 2; }
hipError_t launch_blk_bwd(const BlkArgs& a, int, int grid, hipStream_t) {
    ++g_launches;
    if (grid < 1 || a.cap < 0) fail("block backward launch shape");
    return hipSuccess;
}
hipError_t launch_mx_quant(const MxQuantArgs& a, hipStream_t) {
    ++g_launches;
    region(a.blk_seq, sizeof(int32_t) * (size_t)(a.max_blocks > 0 ? a.max_blocks : 1),
           "quantizer block map outside the workspace");
    return hipSuccess;
}
hipError_t launch_mx_fwd(const MxFwdArgs&, int grid, hipStream_t) {
    ++g_launches;
    if (grid < 1) fail("MXFP8 launch shape");
    return hipSuccess;
}
int mx_fwd_blocks_per_cu() { return 2; }
int probe_threads() { return 256; }
int probe_flop_per_iter() { return 4 * 32 * 32 * 16 * 2 * 4; }
hipError_t launch_probe_mfma(int, int grid, uint64_t* out, float* sink, hipStream_t) {
    ++g_launches;
    region(out, sizeof(uint64_t) * 2 * (size_t)grid, "probe results outside the workspace");
    region(sink, sizeof(float) * 256 * (size_t)grid, "probe sink outside the workspace");
    return hipSuccess;
}

}  // namespace ja

// --- driver ----------------------------------------------------------------------
namespace {

char* const FAKE = reinterpret_cast<char*>(uintptr_t(1) << 40);  // 256-aligned, never dereferenced
const int32_t* const OFF = reinterpret_cast<const int32_t*>(FAKE);

void expect(int got, int want, const char* what) {
    if (got != want) {
        std::fprintf(stderr, "FAIL: %s: status %d, expected %d\n", what, got, want);
        ++g_failures;
    }
}

void sweep_fwd_bwd() {
    const int32_t Bs[] = {0, 1, 7, 2048, 2049, 100000};
    const int64_t Ts[] = {0, 1, 31, 4096, 1 << 20, (int64_t)1 << 30};
    for (int32_t B : Bs)
        for (int32_t H : {1, 8})
            for (int32_t d : {32, 64, 128})
                for (int64_t Tq : Ts)
                    for (int64_t Tk : {(int64_t)0, (int64_t)64 * (B > 0 ? B : 1), Tq, (int64_t)INT32_MAX})
                        for (int dtype : {0, 1})
                            for (int act : {0, 1, 3}) {
                                const size_t fb = ja_fwd_workspace_size(B, H, d, Tq, Tk, act, 1, 0, dtype);
                                if (fb > 0) {
                                    begin_call(FAKE, fb);
                                    expect(jagged_attn_fwd(FAKE, FAKE, FAKE, OFF, OFF, B, H, d, Tq, Tk, act, 1, 0,
                                                           0.1f, dtype, FAKE, (float*)FAKE, FAKE, fb, nullptr),
                                           JA_OK, "forward");
                                    expect(jagged_attn_fwd(FAKE, FAKE, FAKE, OFF, OFF, B, H, d, Tq, Tk, act, 0, 9,
                                                           0.1f, dtype, FAKE, nullptr, FAKE, fb - 1, nullptr),
                                           (B == 0 || Tq == 0) ? JA_OK : JA_ERR_WORKSPACE, "forward, short workspace");
                                }
                                const size_t bb = ja_bwd_workspace_size(B, H, d, Tq, Tk, act, 1, 0, dtype);
                                if (bb > 0) {
                                    for (int gdt : {dtype, 0}) {
                                        begin_call(FAKE, bb);
                                        expect(jagged_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, (float*)FAKE, OFF, OFF,
                                                               B, H, d, Tq, Tk, act, 1, 33, 0.1f, dtype, gdt, FAKE,
                                                               FAKE, FAKE, FAKE, bb, nullptr),
                                               JA_OK, "backward");
                                    }
                                    expect(jagged_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, (float*)FAKE, OFF, OFF, B, H,
                                                           d, Tq, Tk, act, 1, 33, 0.1f, dtype, dtype, FAKE, FAKE,
                                                           FAKE, FAKE, bb - 1, nullptr),
                                           (B == 0 || (Tq == 0 && Tk == 0)) ? JA_OK : JA_ERR_WORKSPACE,
                                           "backward, short workspace");
                                }
                            }
}

void sweep_block_mx_misc() {
    for (int32_t B : {0, 1, 33, 5000})
        for (int64_t T : {(int64_t)0, (int64_t)1, (int64_t)777, (int64_t)1 << 24})
            for (int32_t block : {1, 16, 64, 128, 1024}) {
                const size_t wb = ja_block_attn_workspace_size(B, 4, 128, T, block, 1, 1);
                if (wb == 0) continue;
                begin_call(FAKE, wb);
                expect(jagged_block_attn_fwd(FAKE, FAKE, FAKE, OFF, B, 4, 128, T, block, 1, 0.1f, 1, FAKE, nullptr,
                                             FAKE, wb, nullptr),
                       JA_OK, "block forward");
                begin_call(FAKE, wb);
                expect(jagged_block_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, (float*)FAKE, OFF, B, 4, 128, T, block, 1,
                                             0.1f, 1, FAKE, FAKE, FAKE, FAKE, wb, nullptr),
                       JA_OK, "block backward");
            }
    for (int32_t B : {0, 1, 33, 5000})
        for (int64_t T : {(int64_t)0, (int64_t)5, (int64_t)100000}) {
            const size_t qb = ja_mxfp8_quantize_workspace_size(B, T);
            begin_call(FAKE, qb);
            expect(ja_mxfp8_quantize(FAKE, 1, OFF, B, 2, 128, T, FAKE, FAKE, (int32_t*)FAKE, FAKE, qb, nullptr),
                   JA_OK, "MXFP8 quantize");
            const size_t fb = ja_fwd_mxfp8_workspace_size(B, 2, 128, T, T);
            if (fb == 0) continue;
            begin_call(FAKE, fb);
            expect(jagged_attn_fwd_mxfp8(FAKE, FAKE, OFF, FAKE, FAKE, OFF, FAKE, FAKE, OFF, OFF, B, 2, 128, T, T, 1,
                                         0, 0.1f, FAKE, (float*)FAKE, FAKE, fb, nullptr),
                   JA_OK, "MXFP8 forward");
        }
    // schedule copy-out, tile shapes, profile hooks, probe, status strings
    const size_t sb = ja_fwd_workspace_size(9, 2, 64, 5000, 5000, 0, 1, 0, 1);
    begin_call(FAKE, sb);
    expect(ja_fwd_schedule(OFF, OFF, 9, 2, 64, 5000, 5000, 0, 1, 0, 1, (int32_t*)FAKE, (int32_t*)FAKE, 5000, FAKE,
                           sb, nullptr),
           JA_OK, "schedule");
    int32_t bm = 0, bn = 0;
    expect(ja_fwd_tile_shape(9, 64, 5000, 5000, 0, 1, &bm, &bn), JA_OK, "tile shape");
    expect(ja_validate_offsets(nullptr, 3, 10, nullptr), JA_ERR_INVALID_ARG, "validate offsets");
    ja_set_profile_events(nullptr, nullptr);
    ja_set_profile_events3(nullptr, nullptr, nullptr);
    const size_t pb = ja_probe_mfma_workspace_size();
    begin_call(FAKE, pb);
    int32_t groups = 0, khz = 0;
    int64_t fpg = 0;
    const int st = ja_probe_mfma(10, FAKE, pb, &groups, &fpg, &khz, nullptr);
    if (st != JA_OK && st != JA_ERR_HIP) fail("probe status");  // no device: the clock-rate query fails
    for (int s = -1; s <= 7; ++s)
        if (!ja_status_string((ja_status_t)s) || !*ja_status_string((ja_status_t)s)) fail("status string");
}

}  // namespace

int main() {
    sweep_fwd_bwd();
    sweep_block_mx_misc();
    if (g_failures) {
        std::fprintf(stderr, "%ld failures\n", g_failures);
        return 1;
    }
    std::printf("ok: %ld launches checked\n", g_launches);
    return 0;
}
