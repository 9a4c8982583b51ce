/*
 * ja_oracle.h -- fp64 CPU oracle for jagged attention (test infrastructure).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this library: only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no source with the HIP
 * library and is written from the definitions on the pages, not from any
 * kernel.
 *
 * Source: "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads
 * Foundation Model" (engineering post, indiaaifounders.com copy):
 *   - section "Jagged Sequence Flash Attention": attention computed directly on
 *     variable-length (jagged) sequences, with asymmetric query/key-value
 *     lengths, reaching what padded scaled-dot-product attention reaches
 *     without the padding;
 *   - section "Generalized Dot-Product Attention (GDPA)": two matrix products
 *     with an element-wise activation (GELU or SiLU) in place of softmax,
 *     covering self-attention, PMA and cross-attention;
 *   - section "BlockAttention": sliding-window attention that limits each
 *     token to nearby events.
 *
 * Readings where the pages are silent (each one also listed in the design
 * notes of the repository):
 *   - the pointwise activations are normalised by 1/Lk_b, Lk_b being the key
 *     count of the sequence;
 *   - GELU is the tanh form (the pages name GELU's tanh);
 *   - the ALU-only GELU of the same section (ORA_GELU_TAYLOR) is the Taylor
 *     polynomial of that tanh form about 0 through x^6 (the pages' Taylor
 *     expansion of order 6), used where QK-norm keeps |scale q.k| small: it is
 *     within 1.2e-3 of the tanh form for |x| <= 1;
 *   - causal is top-left aligned: key j is visible to query i iff j <= i;
 *   - a window W > 0 keeps W keys including the query's own position:
 *     causal: 0 <= i - j < W; non-causal: |i - j| < W; W == 0 means no window;
 *   - a row with no visible key outputs 0 (softmax: lse = -inf).
 *
 * Pins: every function here is checked, in the CPU test suite, against
 * library routines (torch scaled_dot_product_attention / autograd in float64
 * on padded dense tensors), closed forms (identical keys, zero queries,
 * constant values, single visible key), invariants (sequence permutation) and
 * central finite differences. The work-list function is pinned by brute-force
 * enumeration.
 */
#ifndef JA_ORACLE_H
#define JA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORA_F32 = 0, ORA_BF16 = 1, ORA_F64 = 2 };
enum { ORA_SOFTMAX = 0, ORA_SILU = 1, ORA_GELU_TANH = 2, ORA_GELU_TAYLOR = 3 };

/* Forward. q: [Tq,H,d], k/v: [Tk,H,d] token-major, element type `dtype`
 * (bf16 given as raw uint16 bits). Offsets: [B+1], non-decreasing from 0.
 * pair_mask: [B*H] bytes, index b*H+h; NULL computes every pair. Rows of
 * unselected pairs are not written. out: [Tq,H,d] doubles; lse: [Tq,H]
 * doubles or NULL (softmax only; GDPA writes NaN there).
 * nthreads <= 0 uses every online core. Returns 0, or -1 on bad arguments. */
int ora_fwd(const void* q, const void* k, const void* v, int dtype,
            const int32_t* q_off, const int32_t* k_off,
            int32_t B, int32_t H, int32_t d,
            int act, int causal, int32_t window, double scale,
            const uint8_t* pair_mask, double* out, double* lse, int nthreads);

/* Backward of the softmax forward (act must be ORA_SOFTMAX) or of the
 * normalised pointwise forward (ORA_SILU / ORA_GELU_TANH / ORA_GELU_TAYLOR). The oracle
 * recomputes its own O and LSE. dout: [Tq,H,d] in `dtype`. Writes out, lse
 * (may be NULL), dq [Tq,H,d], dk and dv [Tk,H,d] for the selected pairs. */
int ora_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
            const int32_t* q_off, const int32_t* k_off,
            int32_t B, int32_t H, int32_t d,
            int act, int causal, int32_t window, double scale,
            const uint8_t* pair_mask, double* out, double* lse,
            double* dq, double* dk, double* dv, int nthreads);

/* Reference work list of (sequence, row-tile) items for a row-tiled pass over
 * a jagged batch: rows of sequence b are `row_off`, columns `col_off`. Each
 * row tile of BM rows has a column range of visible columns (causal / window
 * as above, `transposed` = 1 when rows are keys and columns are queries, as in
 * a key-stationary backward pass); its cost is the number of BN-wide column
 * tiles that range touches. Items are sorted by min(cost, cap) descending,
 * then b ascending, then tile ascending. Writes items[2*n] = b, items[2*n+1]
 * = tile, costs[n] = cost. Returns the item count, or -1 if max_items is too
 * small or an argument is bad. */
int64_t ora_tile_list(const int32_t* row_off, const int32_t* col_off, int32_t B,
                      int32_t BM, int32_t BN, int causal, int32_t window,
                      int transposed, int32_t cap,
                      int32_t* items, int32_t* costs, int64_t max_items);

/* Number of online cores the oracle uses when nthreads <= 0. */
int ora_num_threads(void);

/* The same three functions with a block-diagonal mask ("BlockAttention"
 * section: fixed token blocks, each query block attending only to its own
 * key/value block): block G > 0 additionally requires floor(i/G) == floor(j/G)
 * for query i to see key j (local indices); G == 0 is the functions above. */
int ora_fwd_block(const void* q, const void* k, const void* v, int dtype,
                  const int32_t* q_off, const int32_t* k_off,
                  int32_t B, int32_t H, int32_t d,
                  int act, int causal, int32_t window, int32_t block, double scale,
                  const uint8_t* pair_mask, double* out, double* lse, int nthreads);
int ora_bwd_block(const void* q, const void* k, const void* v, const void* dout, int dtype,
                  const int32_t* q_off, const int32_t* k_off,
                  int32_t B, int32_t H, int32_t d,
                  int act, int causal, int32_t window, int32_t block, double scale,
                  const uint8_t* pair_mask, double* out, double* lse,
                  double* dq, double* dk, double* dv, int nthreads);
int64_t ora_tile_list_block(const int32_t* row_off, const int32_t* col_off, int32_t B,
                            int32_t BM, int32_t BN, int causal, int32_t window, int32_t block,
                            int transposed, int32_t cap,
                            int32_t* items, int32_t* costs, int64_t max_items);

/* MXFP8 ("Mixed Ultra-Low-Precision Training" section: block-scaled FP8
 * attention, one scale per [32, 32] block so that a tensor and its transpose
 * share one quantization). Readings: elements are E4M3 ("fn": largest finite
 * 448, no infinities), scales E8M0 powers of two; a block covers 32 consecutive
 * tokens of one sequence (blocks restart at every sequence start, the last may
 * be short) times 32 consecutive channels of one head; its scale exponent is
 * floor(log2(amax)) - 8 (E4M3's largest exponent), limited to [-127, 127]
 * (-127 for an all-zero block), and each element is x / 2^e clamped to +-448
 * and rounded to the nearest E4M3 value, ties to even.
 * ora_e4m3_encode: nearest E4M3 code of x in [-448, 448]; ora_e4m3_decode: its
 * value (NaN for the NaN codes). */
double ora_e4m3_decode(uint8_t b);
uint8_t ora_e4m3_encode(double x);
/* x [T,H,d] -> x8 [T,H,d] E4M3 codes, scales [NB,H,d/32] (byte = exponent + 127),
 * soff [B+1]: first 32-token block of each sequence (NB = soff[B]). */
int ora_mxfp8_quantize(const void* x, int dtype, const int32_t* off, int32_t B, int32_t H, int32_t d,
                       uint8_t* x8, uint8_t* scales, int32_t* soff);
/* Softmax attention forward on dequantized MXFP8 Q, K, V (K and V share
 * k_soff): S = scale Q K^T, the row max m and sum l = sum_j exp(S_ij - m) of
 * the visible keys, then with pquant the weights exp(S_ij - m) rounded to E4M3
 * at the fixed scale 2^-8 (they are at most 1, so no per-block amax is needed:
 * the softmax's own row max sets the scale) before the product with V;
 * out = sum_j P_ij V_j / l, lse = m + ln l. pquant = 0 gives plain softmax
 * attention on the dequantized tensors. */
int ora_fwd_mxfp8(const uint8_t* q8, const uint8_t* qs, const int32_t* q_soff,
                  const uint8_t* k8, const uint8_t* ks, const int32_t* k_soff,
                  const uint8_t* v8, const uint8_t* vs,
                  const int32_t* q_off, const int32_t* k_off, int32_t B, int32_t H, int32_t d,
                  int causal, int32_t window, double scale, int pquant,
                  const uint8_t* pair_mask, double* out, double* lse, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
