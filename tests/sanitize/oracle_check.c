/* The fp64 oracle (oracle/ja_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer, built with gcc for the CPU. Every buffer is
 * allocated at exactly its documented size, so an access past any of them is
 * reported. Calls every oracle entry point on ragged batches (empty sequences,
 * single tokens, lengths across tile edges, cross-attention lengths) with every
 * activation and mask, fp32 and bf16 inputs, the block-diagonal mask, the tile
 * lists with exactly-sized item buffers, and the MXFP8 quantizer and forward;
 * checks that outputs are finite where defined. Prints "ok" and exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ja_oracle.h"

static int failures = 0;
#define CHECK(c, msg)                             \
    do {                                          \
        if (!(c)) {                               \
            fprintf(stderr, "FAIL: %s\n", msg);   \
            ++failures;                           \
        }                                         \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*: uniform in [0, 1) */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static float nrand(void) { return (float)(urand() + urand() + urand() - 1.5) * 2.0f; }

static uint16_t to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static void* draw(int64_t n, int dtype) {
    void* p = malloc((size_t)(n > 0 ? n : 1) * (dtype == ORA_BF16 ? 2 : 4));
    for (int64_t i = 0; i < n; ++i) {
        const float x = nrand();
        if (dtype == ORA_BF16) ((uint16_t*)p)[i] = to_bf16(x);
        else ((float*)p)[i] = x;
    }
    return p;
}

static int32_t* offsets(const int32_t* len, int32_t B) {
    int32_t* o = malloc(sizeof(int32_t) * (size_t)(B + 1));
    o[0] = 0;
    for (int32_t b = 0; b < B; ++b) o[b + 1] = o[b] + len[b];
    return o;
}

static void run_case(const int32_t* lq, const int32_t* lk, int32_t B, int32_t H, int32_t d, int dtype) {
    int32_t* qo = offsets(lq, B);
    int32_t* ko = offsets(lk, B);
    const int64_t Tq = qo[B], Tk = ko[B];
    void* q = draw(Tq * H * d, dtype);
    void* k = draw(Tk * H * d, dtype);
    void* v = draw(Tk * H * d, dtype);
    void* dout = draw(Tq * H * d, dtype);
    double* out = malloc(sizeof(double) * (size_t)(Tq * H * d + 1));
    double* lse = malloc(sizeof(double) * (size_t)(Tq * H + 1));
    double* dq = malloc(sizeof(double) * (size_t)(Tq * H * d + 1));
    double* dk = malloc(sizeof(double) * (size_t)(Tk * H * d + 1));
    double* dv = malloc(sizeof(double) * (size_t)(Tk * H * d + 1));
    uint8_t* mask = malloc((size_t)(B * H + 1));
    for (int32_t i = 0; i < B * H; ++i) mask[i] = (uint8_t)(i % 3 != 1);
    const int acts[] = {ORA_SOFTMAX, ORA_SILU, ORA_GELU_TANH, ORA_GELU_TAYLOR};
    const int32_t windows[] = {0, 1, 37};
    for (int ai = 0; ai < 4; ++ai)
        for (int causal = 0; causal <= 1; ++causal)
            for (int wi = 0; wi < 3; ++wi)
                for (int block = 0; block <= 16; block += 16) {
                    const int act = acts[ai];
                    const double scale = 1.0 / sqrt((double)d);
                    CHECK(ora_fwd_block(q, k, v, dtype, qo, ko, B, H, d, act, causal, windows[wi], block, scale,
                                        (block ? mask : NULL), out, lse, 3) == 0, "forward");
                    for (int64_t i = 0; i < Tq * H * d; ++i)
                        if (!block || mask[0]) CHECK(isfinite(out[i]) || isnan(out[i]), "forward value");
                    if (dtype == ORA_BF16 && block == 0) {
                        CHECK(ora_bwd_block(q, k, v, dout, dtype, qo, ko, B, H, d, act, causal, windows[wi], 0,
                                            scale, NULL, out, lse, dq, dk, dv, 2) == 0, "backward");
                        for (int64_t i = 0; i < Tq * H * d; ++i) CHECK(isfinite(dq[i]), "dq finite");
                        for (int64_t i = 0; i < Tk * H * d; ++i) CHECK(isfinite(dk[i]) && isfinite(dv[i]), "dk dv");
                    }
                }
    /* reference work lists with exactly-sized buffers */
    for (int t = 0; t <= 1; ++t) {
        const int32_t* ro = t ? ko : qo;
        const int32_t* co = t ? qo : ko;
        int64_t n = 0;
        for (int32_t b = 0; b < B; ++b) n += (ro[b + 1] - ro[b] + 63) / 64;
        int32_t* items = malloc(sizeof(int32_t) * (size_t)(2 * n + 1));
        int32_t* costs = malloc(sizeof(int32_t) * (size_t)(n + 1));
        CHECK(ora_tile_list_block(ro, co, B, 64, 32, 1, 20, 0, t, 511, items, costs, n) == n, "tile list");
        CHECK(ora_tile_list_block(ro, co, B, 64, 32, 0, 0, 16, t, 511, items, costs, n) == n, "block tile list");
        if (n > 0) CHECK(ora_tile_list_block(ro, co, B, 64, 32, 0, 0, 0, t, 511, items, costs, n - 1) == -1,
                         "tile list rejects a short buffer");
        free(items);
        free(costs);
    }
    /* MXFP8 (bf16 inputs, d a multiple of 32) */
    if (dtype == ORA_BF16 && d % 32 == 0) {
        int64_t nbq = 0, nbk = 0;
        for (int32_t b = 0; b < B; ++b) {
            nbq += (lq[b] + 31) / 32;
            nbk += (lk[b] + 31) / 32;
        }
        uint8_t* q8 = malloc((size_t)(Tq * H * d + 1));
        uint8_t* k8 = malloc((size_t)(Tk * H * d + 1));
        uint8_t* v8 = malloc((size_t)(Tk * H * d + 1));
        uint8_t* qs = malloc((size_t)(nbq * H * (d / 32) + 1));
        uint8_t* ks = malloc((size_t)(nbk * H * (d / 32) + 1));
        uint8_t* vs = malloc((size_t)(nbk * H * (d / 32) + 1));
        int32_t* qso = malloc(sizeof(int32_t) * (size_t)(B + 1));
        int32_t* kso = malloc(sizeof(int32_t) * (size_t)(B + 1));
        CHECK(ora_mxfp8_quantize(q, dtype, qo, B, H, d, q8, qs, qso) == 0, "quantize q");
        CHECK(ora_mxfp8_quantize(k, dtype, ko, B, H, d, k8, ks, kso) == 0, "quantize k");
        CHECK(ora_mxfp8_quantize(v, dtype, ko, B, H, d, v8, vs, kso) == 0, "quantize v");
        CHECK(qso[B] == nbq && kso[B] == nbk, "scale offsets");
        for (int pq = 0; pq <= 1; ++pq)
            CHECK(ora_fwd_mxfp8(q8, qs, qso, k8, ks, kso, v8, vs, qo, ko, B, H, d, 1, 0, 1.0 / sqrt((double)d), pq,
                                NULL, out, lse, 2) == 0, "MXFP8 forward");
        free(q8); free(k8); free(v8); free(qs); free(ks); free(vs); free(qso); free(kso);
    }
    for (int c = 0; c < 256; ++c) {
        const double x = ora_e4m3_decode((uint8_t)c);
        if (isfinite(x)) CHECK(ora_e4m3_decode(ora_e4m3_encode(x)) == x, "E4M3 round trip");
    }
    free(q); free(k); free(v); free(dout); free(out); free(lse); free(dq); free(dk); free(dv); free(mask);
    free(qo); free(ko);
}

int main(void) {
    const int32_t lq1[] = {1, 7, 64, 65, 0, 129, 33};
    run_case(lq1, lq1, 7, 2, 32, ORA_BF16);
    run_case(lq1, lq1, 7, 1, 64, ORA_F32);
    const int32_t lq2[] = {200, 1, 0, 77, 130};
    const int32_t lk2[] = {64, 300, 5, 0, 1};
    run_case(lq2, lk2, 5, 3, 64, ORA_BF16);
    run_case(lq2, lk2, 0, 1, 32, ORA_BF16); /* empty batch */
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
