/*
 * jagged_attn.h -- C ABI of the MI355X (gfx950) jagged attention library.
 *
 * What is computed. For a batch of B variable-length ("jagged") sequences stored
 * back to back with no padding, each sequence b and head h computes
 *     out = act(scale * Q K^T, masks) V
 * over its own rows only. The engineering post "GEM Training: How Meta Doubled
 * the Efficiency of Its LLM-Scale Ads Foundation Model" defines the operations:
 *   - "Jagged Sequence Flash Attention" section: FlashAttention run directly on
 *     variable-length jagged tensors addressed per sequence, with asymmetric
 *     query / key-value lengths and a backward pass whose dQ is computed in its
 *     own pass (no atomic dQ accumulation, no recomputation across passes);
 *   - "Generalized Dot-Product Attention (GDPA)" section: the same two matrix
 *     products with an element-wise GELU or SiLU in place of softmax, for
 *     self-attention, cross-attention (long queries, short keys/values) and
 *     pooled multi-head attention (short queries, long keys/values); valid tiles
 *     are enumerated by a software tile scheduler and empty tiles skipped;
 *   - "BlockAttention" section: sliding-window attention that limits each token
 *     to nearby events and skips tiles outside the window, and its block-diagonal
 *     form (jagged_block_attn_fwd / _bwd) where fixed token blocks attend only
 *     within themselves.
 *
 * Conventions this library fixes where the post is silent:
 *   - SiLU(x) = x * sigmoid(x); GELU is the tanh form
 *     0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))); both are normalised by
 *     1/Lk_b, Lk_b being the key count of the sequence (all keys, not the
 *     visible ones). Softmax is normalised by its own row sum.
 *   - causal is top-left aligned: query i (local index) sees key j iff j <= i;
 *   - window W > 0 keeps W keys including the query's own position:
 *     causal: 0 <= i - j < W; non-causal: |i - j| < W. W == 0: no window.
 *   - a row with no visible key gets out = 0 and (softmax) lse = -inf.
 *
 * Layout. Q, out, dQ: [Tq, H, d]; K, V, dK, dV: [Tk, H, d]; token-major, d
 * contiguous, element type `dtype`. lse: [Tq, H] float32, natural log. Offsets
 * are int32 [B+1], non-decreasing, offsets[0] = 0, offsets[B] = T. K and V share
 * k_offsets. Sequence b owns rows [q_offsets[b], q_offsets[b+1]) of Q and
 * [k_offsets[b], k_offsets[b+1]) of K and V.
 *
 * Ownership and asynchrony. Every pointer argument except the host-side size
 * queries is device memory owned by the caller, including the workspace; the
 * library allocates nothing per call and keeps no pointer after returning. All
 * work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 * the call returns without synchronising: inputs must stay valid and outputs
 * untouched until the stream has passed the call. Outputs and the workspace must
 * not share memory with any input or with each other (inputs may share memory
 * with each other): kernels of one call read inputs after others have written
 * outputs (the backward's dK/dV pass reads Q and dO after its dQ pass has written
 * dQ), so overlapping buffers give undefined results. The library does not check
 * this; the Python binding refuses such calls.
 *
 * Errors. Status codes only: no exceptions cross the ABI, nothing aborts or
 * prints. Problems visible on the host (null pointers, unsupported d or dtype,
 * negative window, non-finite scale, misaligned pointers, a workspace that is
 * too small) return before anything is enqueued. Offsets are not read on the
 * host; malformed offsets are undefined behaviour on the device side, and
 * ja_validate_offsets exists to check them (synchronously) in tests.
 */
#ifndef JAGGED_ATTN_H
#define JAGGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    JA_OK = 0,
    JA_ERR_INVALID_ARG = 1,     /* null pointer, bad size, window < 0, scale not finite, misalignment */
    JA_ERR_UNSUPPORTED = 2,     /* d not in {32, 64, 128}, unknown dtype/act, bwd of fp32, Tq or Tk
                                   above 2^31 - 1, or token rows of more than 2^20 elements (H d) */
    JA_ERR_WORKSPACE = 3,       /* workspace smaller than the matching *_workspace_size() */
    JA_ERR_INVALID_OFFSETS = 4, /* ja_validate_offsets found malformed offsets */
    JA_ERR_HIP = 5,             /* a HIP runtime call or kernel launch failed */
    JA_ERR_SCRATCH = 6          /* jagged_attn_fwd_noalloc: the sizes need more workspace than its
                                   fixed device buffer holds */
} ja_status_t;

typedef enum {
    JA_ACT_SOFTMAX = 0,  /* online softmax over the visible keys (JFA) */
    JA_ACT_SILU = 1,     /* x*sigmoid(x), times 1/Lk_b (GDPA) */
    JA_ACT_GELU_TANH = 2,  /* tanh-form GELU, times 1/Lk_b (GDPA) */
    JA_ACT_GELU_TAYLOR = 3 /* ALU-only GELU, times 1/Lk_b (GDPA): the Taylor polynomial of the tanh
                              form about 0 through x^6, x/2 + k2 x^2 + k4 x^4 + k6 x^6 with
                              c = sqrt(2/pi): k2 = c/2, k4 = (0.044715 c - c^3/3)/2,
                              k6 = (2 c^5/15 - 0.044715 c^3)/2; no transcendental instruction.
                              Within 1.2e-3 of JA_ACT_GELU_TANH for |scale q.k| <= 1, the range
                              unit-norm (QK-normed) queries and keys give with scale <= 1;
                              diverges from it beyond about |x| = 1.5. */
} ja_act_t;

typedef enum {
    JA_F32 = 0,  /* fp32 in, fp32 out, fp32 matrix-core products */
    JA_BF16 = 1  /* bf16 in, bf16 out, fp32 accumulation */
} ja_dtype_t;

/* Bytes of device workspace jagged_attn_fwd needs for these sizes. Host only. */
size_t ja_fwd_workspace_size(int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                             int32_t act, int32_t causal, int32_t window, int32_t dtype);

/* Forward (the whole hot path: tile scheduling, then the fused attention kernel).
 *   q [Tq,H,d], k/v [Tk,H,d]: inputs, 16-byte aligned.
 *   q_offsets, k_offsets: device int32 [B+1].
 *   B >= 0, H >= 1, d in {32, 64, 128}; Tq, Tk: first dimensions of q and k.
 *   act: ja_act_t; causal: 0/1; window >= 0 (0 = none); scale: finite, applied
 *   to Q K^T before the activation (usually 1/sqrt(d)).
 *   out [Tq,H,d]: written for every row of every sequence.
 *   lse [Tq,H] fp32: softmax log-sum-exp per row, natural log; may be NULL;
 *   ignored for SiLU/GELU.
 *   workspace: at least ja_fwd_workspace_size() bytes, 16-byte aligned; its
 *   contents on entry do not matter and are clobbered. */
ja_status_t jagged_attn_fwd(const void* q, const void* k, const void* v,
                            const int32_t* q_offsets, const int32_t* k_offsets,
                            int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                            int32_t act, int32_t causal, int32_t window, float scale,
                            int32_t dtype, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Size of the fixed per-GPU device buffer jagged_attn_fwd_noalloc uses as its workspace. */
#define JA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/* jagged_attn_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, results and errors as jagged_attn_fwd, without the workspace: it uses
 * a fixed file-scope device buffer of JA_NOALLOC_SCRATCH_BYTES (8 MiB) that every
 * GPU the library runs on holds until the process ends; its address is looked up
 * on the first call with each device current. Calls whose
 * ja_fwd_workspace_size() exceeds that return JA_ERR_SCRATCH before anything is
 * enqueued (8 MiB holds a work list of about 260,000 (sequence, tile) items of 32
 * bytes, ceil(Tq / BM) + B of them: some 33 million query tokens at BM = 128, see
 * ja_fwd_tile_shape). No call allocates or
 * frees anything. All calls on one GPU share the buffer, and each call's contents
 * last until the next one: calls that overlap on one GPU (several streams or host
 * threads) race and must be serialised by the caller. Nothing needs clearing
 * between calls: each call's tile scheduler writes everything its attention
 * kernel reads. */
ja_status_t jagged_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                    const int32_t* q_offsets, const int32_t* k_offsets,
                                    int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                                    int32_t act, int32_t causal, int32_t window, float scale,
                                    int32_t dtype, void* out, float* lse, void* stream);

/* Bytes of device workspace jagged_attn_bwd needs. Host only. */
size_t ja_bwd_workspace_size(int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                             int32_t act, int32_t causal, int32_t window, int32_t dtype);

/* Backward of jagged_attn_fwd for dtype JA_BF16 and every act ("Jagged Sequence
 * Flash Attention" section of the GEM training post: dQ in its own pass, no
 * atomics; "Generalized Dot-Product Attention (GDPA)" section for SiLU / GELU).
 * Writes dq once per row from a query-stationary pass, then dk and dv once per
 * row from a key-stationary pass; no atomics on any gradient.
 *   act == JA_ACT_SOFTMAX: needs the forward's out and lse (same scale); Di =
 *     rowsum(dO * O) is computed inside the dQ pass into the workspace.
 *   act == JA_ACT_SILU / _GELU_TANH / _GELU_TAYLOR: with Z = scale Q K^T, P = act(Z)/Lk
 *     and dS = act'(Z) * (dO V^T) / Lk; out and lse are not read and may be
 *     NULL.
 *   dout [Tq,H,d]: upstream gradient; dq [Tq,H,d], dk/dv [Tk,H,d]: outputs,
 *   every row written (rows no query sees get zeros), of element type
 *   grad_dtype: dtype (bf16) or JA_F32. fp32 gradients keep the fp32 accumulators
 *   unrounded, for callers that accumulate gradients in fp32 or need results
 *   below bf16's resolution (a gradient of magnitude 4 to 8 is otherwise stored
 *   to within 2^-6); anything else returns JA_ERR_UNSUPPORTED. */
ja_status_t jagged_attn_bwd(const void* q, const void* k, const void* v,
                            const void* out, const void* dout, const float* lse,
                            const int32_t* q_offsets, const int32_t* k_offsets,
                            int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                            int32_t act, int32_t causal, int32_t window, float scale,
                            int32_t dtype, int32_t grad_dtype, void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace jagged_block_attn_fwd and jagged_block_attn_bwd
 * need (either call). Host only; 0 for invalid sizes or a block that is not a
 * power of two. */
size_t ja_block_attn_workspace_size(int32_t B, int32_t H, int32_t d, int64_t T, int32_t block,
                                    int32_t causal, int32_t dtype);

/* Block-diagonal self-attention ("BlockAttention" section of the GEM training
 * post: the sequence is cut into fixed blocks of tokens and each query block
 * attends only to the keys and values of its own block, which turns attention
 * into independent small problems). Softmax only; one offsets array serves
 * queries, keys and values (self-attention, Tq = Tk = T).
 *   block: tokens per block, a power of two >= 1; query i (local index) sees key
 *   j iff i / block == j / block (integer division), and with causal also j <= i.
 *   Blocks restart at every sequence start; the last block of a sequence may be
 *   shorter than `block`.
 *   Runs the forward kernel of jagged_attn_fwd under the block mask: tiles off
 *   the diagonal blocks are never scheduled, and with block <= 64 every row's
 *   keys lie in one 64-key stage, so the online softmax takes a single step.
 *   lse [T,H] fp32 may be NULL (then not written; the backward of blocks of at
 *   most 64 tokens does not need it).
 * Everything else (layout, scale, alignment, ownership, errors) is as for
 * jagged_attn_fwd with act = JA_ACT_SOFTMAX and window = 0. workspace: at least
 * ja_block_attn_workspace_size() bytes. A block that is not a power of two
 * returns JA_ERR_INVALID_ARG. */
ja_status_t jagged_block_attn_fwd(const void* q, const void* k, const void* v,
                                  const int32_t* offsets, int32_t B, int32_t H, int32_t d,
                                  int64_t T, int32_t block, int32_t causal, float scale,
                                  int32_t dtype, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Backward of jagged_block_attn_fwd (dtype JA_BF16). For block <= 64 one fused
 * kernel per 64-token tile and head recomputes the block's softmax, takes Di as
 * sum_j P_ij dP_ij, and writes dq, dk and dv once each: out and lse are not read
 * and may be NULL. Larger blocks run jagged_attn_bwd's two passes under the
 * block mask and need the forward's out and lse. workspace: at least
 * ja_block_attn_workspace_size() bytes. */
ja_status_t jagged_block_attn_bwd(const void* q, const void* k, const void* v,
                                  const void* out, const void* dout, const float* lse,
                                  const int32_t* offsets, int32_t B, int32_t H, int32_t d,
                                  int64_t T, int32_t block, int32_t causal, float scale,
                                  int32_t dtype, void* dq, void* dk, void* dv,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* MXFP8 ("Mixed Ultra-Low-Precision Training" section of the GEM training post:
 * attention on block-scaled FP8 with one scale per [32, 32] block, so a tensor
 * and its transpose share one quantization). Format (OCP MX): E4M3 elements
 * ("fn": largest finite 448), E8M0 scales (byte = exponent + 127). A block is 32
 * consecutive tokens of one sequence (blocks restart at every sequence start,
 * the last may be short) by 32 consecutive channels of one head; its exponent
 * is floor(log2(amax)) - 8 limited to [-127, 127] (-127 for an all-zero block),
 * and each element is x / 2^e clamped to +-448, rounded to nearest even. */

/* Bytes of workspace ja_mxfp8_quantize needs. Host only. */
size_t ja_mxfp8_quantize_workspace_size(int32_t B, int64_t T);

/* Quantizes x (JA_BF16 [T,H,d], d a multiple of 32, 16-byte aligned) to
 *   x8 [T,H,d] E4M3 codes (16-byte aligned),
 *   scales [NB,H,d/32] E8M0 bytes, sized for NB = ceil(T/32) + B rows (the first
 *   scale_offsets[B] rows are written),
 *   scale_offsets [B+1] int32: first scale row of each sequence (written).
 * Enqueued on stream, no synchronisation. */
ja_status_t ja_mxfp8_quantize(const void* x, int32_t dtype, const int32_t* offsets,
                              int32_t B, int32_t H, int32_t d, int64_t T,
                              void* x8, void* scales, int32_t* scale_offsets,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace jagged_attn_fwd_mxfp8 needs (0 for unsupported sizes). */
size_t ja_fwd_mxfp8_workspace_size(int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk);

/* Softmax attention forward on MXFP8 inputs as ja_mxfp8_quantize writes them
 * (K and V share k_scale_offsets), d = 128. Both products run on the MX-scaled
 * FP8 matrix cores with the blocks' scales; the softmax keeps an exact running
 * max, so every weight exp(s - m) is at most 1, and is rounded to E4M3 at the
 * fixed scale 2^-8 before the product with V (the row max sets its scale); the
 * normaliser sums the unrounded weights. out [Tq,H,d] is bf16, lse [Tq,H] fp32
 * natural log (may be NULL). Masks, offsets, scale, ownership and errors as
 * jagged_attn_fwd (act = softmax); d other than 128 returns JA_ERR_UNSUPPORTED. */
ja_status_t jagged_attn_fwd_mxfp8(const void* q8, const void* q_scales, const int32_t* q_scale_offsets,
                                  const void* k8, const void* k_scales, const int32_t* k_scale_offsets,
                                  const void* v8, const void* v_scales,
                                  const int32_t* q_offsets, const int32_t* k_offsets,
                                  int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                                  int32_t causal, int32_t window, float scale,
                                  void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Runs only the tile scheduler that jagged_attn_fwd runs first ("software tile
 * scheduling for jagged tensors", GDPA section) and copies its work list out:
 * items (device int32 [2*max_items]) receives (sequence, query-tile) pairs in the
 * order the persistent attention grid consumes them (each pair expands to H
 * work items, head fastest); count (device int32 [1]) receives the number of
 * pairs. Pairs are ordered by min(cost, 511) descending, then sequence, then
 * tile ascending, cost being the number of key tiles the query tile visits.
 * Returns JA_ERR_INVALID_ARG if max_items < ceil(Tq/BM) + B (BM from
 * ja_fwd_tile_shape). */
ja_status_t ja_fwd_schedule(const int32_t* q_offsets, const int32_t* k_offsets,
                            int32_t B, int32_t H, int32_t d, int64_t Tq, int64_t Tk,
                            int32_t act, int32_t causal, int32_t window, int32_t dtype,
                            int32_t* items, int32_t* count, int64_t max_items,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Tile shape the forward uses for these sizes: bm query rows per work item, bn
 * keys per scheduler cost unit. The layout, and so the shape, depends only on
 * B, d, Tq, Tk, act and dtype: short queries (Tq <= 48 B) take 32-row items;
 * short keys with long queries (Tk <= 64 B and Tq >= 512 B, bf16) take items of
 * four consecutive 128-row query tiles that share one resident key/value stage;
 * everything else 128-row items. Host only; returns JA_ERR_UNSUPPORTED for
 * unsupported d / dtype / act. */
ja_status_t ja_fwd_tile_shape(int32_t B, int32_t d, int64_t Tq, int64_t Tk, int32_t act, int32_t dtype,
                              int32_t* bm, int32_t* bn);

/* Checks offsets on the device (non-decreasing, [0] == 0, [B] == T) and waits
 * for the result: synchronous, meant for tests and debugging. Uses no
 * workspace. Returns JA_OK or JA_ERR_INVALID_OFFSETS. */
ja_status_t ja_validate_offsets(const int32_t* offsets, int32_t B, int64_t T, void* stream);

/* Profiling aid. While set (non-NULL), each jagged_attn_fwd / jagged_attn_bwd
 * call made from this host thread records the caller's hipEvent_t `before` on its
 * stream immediately before the first attention kernel (after the scheduler) and
 * `after` immediately after the last one, so that the elapsed time between them is
 * the attention kernels' own duration. Pass NULL, NULL to stop. The events are
 * owned by the caller and must outlive the calls that record them. */
void ja_set_profile_events(void* before, void* after);

/* As ja_set_profile_events, and jagged_attn_bwd also records `mid` between its
 * dQ pass and its dK/dV pass (mid may be NULL), so each pass can be timed alone. */
void ja_set_profile_events3(void* before, void* mid, void* after);

/* Machine probe, a measurement aid outside the attention path: one workgroup of
 * four waves per compute unit (one wave per SIMD) issues `iters` rounds of four
 * independent 32x32x16 bf16 matrix products, with no memory traffic in its loop,
 * so its duration gives the matrix-core rate the GPU sustains, and the shader
 * clock it sustains meanwhile. Writes, per workgroup g, the shader-clock cycles
 * and the constant-rate real-time counter ticks of the loop as uint64 at
 * workspace[2 g] and workspace[2 g + 1] (device memory, at least
 * ja_probe_mfma_workspace_size() bytes, 16-byte aligned; the rest is scratch).
 * Host outputs: *groups = workgroups launched (the compute-unit count),
 * *flop_per_group = matrix flop each performs, *wallclock_khz = the real-time
 * counter's rate. Enqueued on stream, no synchronisation. */
size_t ja_probe_mfma_workspace_size(void);
ja_status_t ja_probe_mfma(int32_t iters, void* workspace, size_t workspace_bytes, int32_t* groups,
                          int64_t* flop_per_group, int32_t* wallclock_khz, void* stream);

/* Static string for a status code. */
const char* ja_status_string(ja_status_t status);

/* Library version, as major*10000 + minor*100 + patch. */
int32_t ja_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JAGGED_ATTN_H */
