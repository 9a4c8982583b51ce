"""GPU parity of the jagged attention forward against the fp64 oracle.

Every case calls the HIP library through its C ABI (Python binding) and compares
element by element with the oracle on the same seeded inputs:
  * small ragged batches spanning several tiles and ragged tails, every mask and
    activation, d in {32, 64, 128}, bf16 and fp32, both kernel layouts;
  * the five named workloads at full size, every (sequence, head) pair, held to
    the strict bf16 bound (fp32 for the first);
  * closed forms (zero queries under SiLU/GELU give exactly 0; identical keys give
    the mean of the visible values), bitwise invariance to sequence order,
    bitwise run-to-run determinism, untouched guard bands around the outputs;
  * the device tile scheduler against the oracle's reference work list (exact).
"""
import math

import numpy as np
import pytest
import torch

import jagged_attention_recsys_amd as ja
import oracle
from jagged_attention_recsys_amd import workloads as W
from _parity import compare, rows_of_pairs, say, term_sums, to_dev, to_host64

pytestmark = pytest.mark.gpu

GUARD = 3


def run_fwd(w, act=None, causal=None, window=None, guard=True):
    act = w.act if act is None else act
    causal = w.causal if causal is None else causal
    window = w.window if window is None else window
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    qo, ko = to_dev(w.q_offsets), to_dev(w.k_offsets)
    Tq = q.shape[0]
    out_full = torch.full((Tq + 2 * GUARD, w.H, w.d), float("nan"), dtype=q.dtype, device=q.device)
    lse_full = torch.full((Tq + 2 * GUARD, w.H), float("nan"), dtype=torch.float32, device=q.device)
    out = out_full[GUARD:GUARD + Tq]
    lse = lse_full[GUARD:GUARD + Tq] if act == "softmax" else None
    ja.jagged_attn_fwd(q, k, v, qo, ko, act=act, causal=causal, window=window, scale=w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    if guard:
        assert torch.isnan(out_full[:GUARD].float()).all() and torch.isnan(out_full[GUARD + Tq:].float()).all()
        assert torch.isnan(lse_full[:GUARD]).all() and torch.isnan(lse_full[GUARD + Tq:]).all()
    return out, lse


def check_against_oracle(w, act, causal, window, pair_mask=None, what="", bounds=False, report=False,
                         mean_rounding=False):
    """Strict bf16 / fp32 bound on every compared element. bounds: the edge-case batches
    (rows with few visible keys) pass their term sums, so that elements whose own bf16
    rounding bound exceeds half the tolerance are held to that bound instead."""
    say(f"[fwd] {what} B={w.B} H={w.H} d={w.d} Tq={w.q.shape[0]} Tk={w.k.shape[0]} {w.dtype} act={act} "
        f"causal={causal} window={window}")
    out, lse = run_fwd(w, act, causal, window)
    ref_out, ref_lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, act, causal, window, w.scale,
                                  pair_mask=pair_mask)
    sel = rows_of_pairs(w.q_offsets, w.H, pair_mask)
    got = to_host64(out)
    terms = term_sums(w, act, causal, window, pair_mask=pair_mask) if bounds and w.dtype == "bf16" else None
    stats = compare(got, ref_out, w.dtype, f"out {what}", sel, terms=terms, report=report,
                    mean_rounding=mean_rounding)
    if act == "softmax":
        gl = to_host64(lse)
        fin = np.isfinite(ref_lse) & sel
        assert np.array_equal(np.isneginf(gl) & sel, np.isneginf(ref_lse) & sel), "lse -inf rows differ"
        if fin.any():
            assert np.max(np.abs(gl[fin] - ref_lse[fin])) < 1e-3 * max(1.0, np.max(np.abs(ref_lse[fin])))
    say(f"      ok {stats}")
    return out, lse


RAGGED = [1, 7, 64, 65, 127, 128, 129, 300, 0, 513]
MASKS = [("softmax", False, 0), ("softmax", True, 0), ("softmax", True, 37), ("softmax", False, 50),
         ("silu", False, 0), ("gelu", True, 0), ("silu", True, 100), ("gelu", False, 3)]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("act,causal,window", MASKS)
def test_ragged_self_attention_bf16(d, act, causal, window):
    w = W.make_case(RAGGED, H=2, d=d, dtype=W.BF16, seed=d + window)
    check_against_oracle(w, act, causal, window, what="ragged-self", bounds=True)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("act,causal,window", [("softmax", False, 0), ("softmax", True, 5), ("silu", False, 0),
                                               ("gelu", True, 20)])
def test_ragged_cross_attention_bf16(d, act, causal, window):
    lq = [200, 1, 0, 77, 130, 129]
    lk = [64, 300, 5, 0, 1, 257]
    w = W.make_case(lq, lk, H=3, d=d, dtype=W.BF16, seed=7 * d + window)
    check_against_oracle(w, act, causal, window, what="ragged-cross", bounds=True)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("act,causal,window", [("softmax", False, 0), ("softmax", True, 9), ("silu", False, 0),
                                               ("gelu", False, 0)])
def test_ragged_fp32(d, act, causal, window):
    w = W.make_case([5, 130, 64, 0, 200], H=2, d=d, dtype=W.F32, seed=11 * d)
    check_against_oracle(w, act, causal, window, what="ragged-fp32")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("act,causal,window", [("softmax", False, 0), ("softmax", True, 0), ("gelu", False, 0),
                                               ("silu", True, 40)])
def test_short_queries_split_layout(d, act, causal, window):
    rng = np.random.default_rng(d)
    B = 23
    lq = rng.integers(0, 41, size=B)
    lk = rng.integers(0, 700, size=B)
    lk[0], lk[1] = 0, 1
    w = W.make_case(lq, lk, H=2, d=d, dtype=W.BF16, seed=d + 1)
    bm, bn = ja.fwd_tile_shape(w.B, d, w.q.shape[0], w.k.shape[0], act)
    assert bm == 32, "short-query batch should take the split layout"
    check_against_oracle(w, act, causal, window, what="split", bounds=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("act,causal,window", [("softmax", True, 0), ("softmax", False, 300), ("silu", True, 0),
                                               ("gelu", False, 0)])
def test_mixed_batch_long_queries_split_layout(d, act, causal, window):
    # The layout follows from the batch's totals: a few long query sequences among
    # many short ones keep the mean query length short, so the long ones also run
    # through the split layout's 32-row items (query tiles far past the first,
    # diagonal and window stages across many key slices, a ragged last tile).
    rng = np.random.default_rng(7 * d + window)
    lq = rng.integers(0, 9, size=100)
    lk = rng.integers(0, 400, size=100)
    lq[5], lk[5] = 1500, 1500  # self-attention-like
    lq[40], lk[40] = 1111, 1700  # Lq != Lk
    lq[41], lk[41] = 700, 0  # no keys
    w = W.make_case(lq, lk, H=2, d=d, dtype=W.BF16, seed=d + window)
    bm, bn = ja.fwd_tile_shape(w.B, d, w.q.shape[0], w.k.shape[0], act)
    assert bm == 32, "mean query length <= 48 should take the split layout"
    check_against_oracle(w, act, causal, window, what="mixed-split", bounds=True)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("act,causal,window", [("silu", False, 0), ("gelu", False, 0), ("softmax", False, 0),
                                               ("softmax", True, 0), ("silu", True, 30), ("softmax", False, 50)])
def test_short_keys_chunked_layout(d, act, causal, window):
    # Mean key length <= 64 with mean query length >= 512: items of four 128-row
    # query tiles. Sequences whose keys fit one stage (Lk <= 64) keep it resident
    # for the whole item; Lk = 300 crosses stages and takes the streaming path;
    # partial chunks, single rows, empty queries and empty keys are included.
    lq = [1100, 1, 0, 512, 513, 640, 2049, 700]
    lk = [64, 5, 3, 0, 1, 64, 63, 300]
    w = W.make_case(lq, lk, H=2, d=d, dtype=W.BF16, seed=5 * d + window)
    bm, bn = ja.fwd_tile_shape(w.B, d, w.q.shape[0], w.k.shape[0], act)
    assert (bm, bn) == (512, 64), "short-key batch should take the chunked layout"
    check_against_oracle(w, act, causal, window, what="chunked", bounds=True)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 100)])
def test_peaky_softmax_large_logits(causal, window):
    # Scale 1 at d = 128: scores with a standard deviation near 11 and row maxima near
    # 35, so the weights are nearly one-hot, the running max rises in large steps and
    # most weights underflow.
    w = W.make_case([300, 700, 64, 1], H=2, d=128, dtype=W.BF16, seed=77 + window)
    w.attn_scale = 1.0
    check_against_oracle(w, "softmax", causal, window, what="peaky")


def test_workload1_fp32_softmax_and_silu():
    w = W.workload(1)
    check_against_oracle(w, "softmax", False, 0, what="w1 fwd", report=True)
    check_against_oracle(w, "silu", False, 0, what="w1 fwd silu", report=True)


# Sliding-window batches (bf16, d = 128) pop from eight per-XCD queues, queue q holding
# items 8k + q of the list. Few items leave queues empty from the start, and item counts
# that are not a multiple of eight give queues of different lengths, so workgroups steal
# from other queues and finish when every queue is empty.
WINDOW_QUEUE_CASES = [([5], 1), ([130, 7, 300], 3), ([1000], 2), ([64] * 9 + [129], 1), ([2000, 3], 5)]


@pytest.mark.parametrize("lq,H", WINDOW_QUEUE_CASES)
@pytest.mark.parametrize("window", [37, 300])
def test_window_queues_few_items(lq, H, window):
    w = W.make_case(lq, None, H=H, d=128, dtype=W.BF16, seed=sum(lq) + H + window)
    check_against_oracle(w, "softmax", True, window, what=f"queues {len(lq)} seqs", bounds=True)


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_full_workloads_every_pair(n):
    # The whole batch, every (sequence, head) pair, element by element, strict.
    say(f"[fwd] generating workload {n}")
    w = W.workload(n)
    check_against_oracle(w, w.act, w.causal, w.window, what=f"w{n} fwd", report=True)


@pytest.mark.parametrize("act", ["silu", "gelu"])
def test_zero_queries_give_exact_zero(act):
    w = W.make_case([100, 3, 260], [70, 500, 1], H=2, d=128, dtype=W.BF16, seed=5)
    w.q[:] = 0
    out, _ = run_fwd(w, act, False, 0)
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 40)])
def test_identical_keys_give_mean_of_visible_values(causal, window):
    lq = [150, 9, 300]
    w = W.make_case(lq, H=2, d=64, dtype=W.BF16, seed=6)
    w.k[:] = w.k[0, 0]
    out, _ = run_fwd(w, "softmax", causal, window)
    got = to_host64(out)
    v = W.bf16_bits_to_f32(w.v).astype(np.float64)
    for b, L in enumerate(lq):
        qo = w.q_offsets[b]
        for i in range(L):
            lo = 0 if window == 0 else max(0, i - window + 1)
            hi = i + 1 if causal else (L if window == 0 else min(L, i + window))
            expect = v[qo + lo:qo + hi].mean(axis=0)
            assert np.max(np.abs(got[qo + i] - expect)) < 2e-2


@pytest.mark.parametrize("act,causal,window", [("softmax", True, 0), ("silu", False, 0), ("softmax", False, 70)])
def test_sequence_permutation_is_bitwise_invariant(act, causal, window):
    lq = np.array([300, 0, 129, 64, 17, 700])
    w = W.make_case(lq, H=2, d=128, dtype=W.BF16, seed=8)
    out, lse = run_fwd(w, act, causal, window)
    perm = [3, 5, 0, 2, 1, 4]
    rows = np.concatenate([np.arange(w.q_offsets[b], w.q_offsets[b + 1]) for b in perm]).astype(np.int64)
    wp = W.Workload("perm", w.q[rows], w.k[rows], w.v[rows], W.offsets_from_lengths(lq[perm]),
                    W.offsets_from_lengths(lq[perm]), w.H, w.d, w.dtype)
    out2, lse2 = run_fwd(wp, act, causal, window)
    idx = torch.from_numpy(rows).cuda()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)[idx])
    if lse is not None:
        assert torch.equal(lse2, lse[idx])


def test_runs_are_bitwise_deterministic():
    w = W.workload(2)
    out1, lse1 = run_fwd(w)
    out2, lse2 = run_fwd(w)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)


def test_empty_keys_and_empty_rows():
    # every sequence has zero keys: outputs 0, lse -inf
    w = W.make_case([5, 40], [0, 0], H=2, d=64, dtype=W.BF16, seed=9)
    out, lse = run_fwd(w, "softmax", False, 0)
    assert torch.count_nonzero(out).item() == 0 and torch.isneginf(lse).all()
    # more queries than keys under a causal window: late rows see nothing
    w = W.make_case([300], [20], H=1, d=64, dtype=W.BF16, seed=10)
    check_against_oracle(w, "softmax", True, 8, what="lq>lk")
    out, lse = run_fwd(w, "softmax", True, 8)
    assert torch.isneginf(lse[27:]).all() and torch.count_nonzero(out[27:]).item() == 0
    # single-token batch
    w = W.make_case([1], H=1, d=32, dtype=W.BF16, seed=12)
    check_against_oracle(w, "softmax", True, 0, what="single")


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_schedule_matches_reference_work_list(n):
    w = W.workload(n)
    Tq, Tk = w.q.shape[0], w.k.shape[0]
    items = ja.fwd_schedule(to_dev(w.q_offsets), to_dev(w.k_offsets), w.H, w.d, Tq, Tk, w.act, w.causal,
                            w.window).cpu().numpy()
    bm, bn = ja.fwd_tile_shape(w.B, w.d, Tq, Tk, w.act)
    ref, _ = oracle.tile_list(w.q_offsets, w.k_offsets, bm, bn, w.causal, w.window, cap=511)
    assert np.array_equal(items, ref)


def test_schedule_small_cases_with_cap():
    rng = np.random.default_rng(3)
    for causal, window in [(False, 0), (True, 0), (True, 100), (False, 30)]:
        lq = rng.integers(0, 2000, size=40)
        lq[3] = 40000  # exceeds the 511 cost cap
        w = W.make_case(lq, H=1, d=32, dtype=W.BF16, seed=1)
        Tq = int(w.q_offsets[-1])
        items = ja.fwd_schedule(to_dev(w.q_offsets), to_dev(w.k_offsets), 1, 32, Tq, Tq, "softmax", causal,
                                window).cpu().numpy()
        bm, bn = ja.fwd_tile_shape(w.B, 32, Tq, Tq, "softmax")
        ref, _ = oracle.tile_list(w.q_offsets, w.k_offsets, bm, bn, causal, window, cap=511)
        assert np.array_equal(items, ref)


@pytest.mark.parametrize("B", [2048, 2049, 5000])
def test_schedule_many_sequences(B):
    # Up to 2048 sequences the scheduler keeps its per-sequence tables in LDS;
    # beyond that it reads them from global memory. Both orders must match.
    rng = np.random.default_rng(B)
    lq = rng.integers(0, 700, size=B)
    lk = rng.integers(0, 700, size=B)
    qo, ko = W.offsets_from_lengths(lq), W.offsets_from_lengths(lk)
    Tq, Tk = int(qo[-1]), int(ko[-1])
    for causal, window in [(True, 0), (False, 90)]:
        items = ja.fwd_schedule(to_dev(qo), to_dev(ko), 2, 64, Tq, Tk, "softmax", causal, window).cpu().numpy()
        bm, bn = ja.fwd_tile_shape(B, 64, Tq, Tk, "softmax")
        ref, _ = oracle.tile_list(qo, ko, bm, bn, causal, window, cap=511)
        assert np.array_equal(items, ref)


def test_validate_offsets():
    good = torch.tensor([0, 3, 3, 10], dtype=torch.int32, device="cuda")
    assert ja.validate_offsets(good, 10)
    assert not ja.validate_offsets(good, 11)
    bad = torch.tensor([0, 5, 3, 10], dtype=torch.int32, device="cuda")
    assert not ja.validate_offsets(bad, 10)
