"""GPU parity of the jagged attention backward against the fp64 oracle.

Softmax: the HIP forward produces out and lse (as a training step would), the HIP
backward then produces dQ, dK and dV; the oracle computes all three from its own
fp64 forward. Pointwise SiLU / GELU: the backward reads neither out nor lse (both
are passed as None). Cases: ragged batches spanning several tiles with every
mask, d in {32, 64, 128}, asymmetric lengths, the full sliding-window workload
and the SiLU cross-attention and GELU pooled workloads with every (sequence,
head) pair at the strict bound, a closed form (identical keys give dQ = 0), keys no query sees
(zero gradients), bitwise determinism and sequence-order invariance, and guard
bands around every gradient.
"""
import numpy as np
import pytest
import torch

import jagged_attention_recsys_amd as ja
import oracle
from jagged_attention_recsys_amd import workloads as W
from _parity import (compare, rows_of_pairs, say, softmax_grad_terms_at, stored_out_terms, term_sums, to_dev,
                     to_host64)

from test_gpu_fwd import check_against_oracle

pytestmark = pytest.mark.gpu

GUARD = 2


def guarded(shape, dtype):
    full = torch.full((shape[0] + 2 * GUARD,) + tuple(shape[1:]), float("nan"), dtype=dtype, device="cuda")
    return full, full[GUARD:GUARD + shape[0]]


def run_fwd_bwd(w, causal, window, dout=None, act="softmax", grad_dtype=None):
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    qo, ko = to_dev(w.q_offsets), to_dev(w.k_offsets)
    if act == "softmax":
        out, lse = ja.jagged_attn_fwd(q, k, v, qo, ko, act=act, causal=causal, window=window, scale=w.scale)
    else:
        out = lse = None  # the pointwise backward needs neither
    do = to_dev(w.dout if dout is None else dout)
    gdt = q.dtype if grad_dtype is None else grad_dtype
    fq, dq = guarded(q.shape, gdt)
    fk, dk = guarded(k.shape, gdt)
    fv, dv = guarded(v.shape, gdt)
    ja.jagged_attn_bwd(q, k, v, out, do, lse, qo, ko, act=act, causal=causal, window=window, scale=w.scale,
                       dq=dq, dk=dk, dv=dv, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    for f, n in ((fq, q.shape[0]), (fk, k.shape[0]), (fv, v.shape[0])):
        assert torch.isnan(f[:GUARD].float()).all() and torch.isnan(f[GUARD + n:].float()).all(), "guard band"
    return dq, dk, dv


def check(w, causal, window, pair_mask=None, what="", act="softmax", bounds=False, report=False,
          mean_rounding=False):
    """Strict bf16 bound on every gradient element. The pointwise backward is also held to
    its per-element rounding bound everywhere (its gradients are unnormalised sums over
    up to Lq terms). bounds (softmax): the edge-case batches pass their term sums, so that
    elements whose own bf16 rounding bound exceeds half the tolerance are held to it."""
    say(f"[bwd] {what} act={act} B={w.B} H={w.H} d={w.d} Tq={w.q.shape[0]} Tk={w.k.shape[0]} causal={causal} "
        f"window={window}")
    dq, dk, dv = run_fwd_bwd(w, causal, window, act=act)
    _, _, rq, rk, rv = oracle.bwd(w.q, w.k, w.v, w.dout, w.q_offsets, w.k_offsets, act, causal, window,
                                  w.scale, pair_mask=pair_mask)
    selq = rows_of_pairs(w.q_offsets, w.H, pair_mask)
    selk = rows_of_pairs(w.k_offsets, w.H, pair_mask)
    pointwise = act != "softmax"
    tq = tk = tv = None
    if bounds or pointwise:
        _, tq, tk, tv = term_sums(w, act, causal, window, pair_mask=pair_mask, grads=True)
    stats = {}
    for name, got, ref, terms, sel in (("dq", dq, rq, tq, selq), ("dk", dk, rk, tk, selk), ("dv", dv, rv, tv, selk)):
        stats[name] = compare(to_host64(got), ref, w.dtype, f"{what} {name}", sel, terms=terms, bounded=pointwise,
                              report=report, mean_rounding=mean_rounding)
    say(f"      ok {stats}")


def case(lq, lk=None, H=2, d=64, seed=0):
    return W.make_case(lq, lk, H=H, d=d, dtype=W.BF16, seed=seed, with_dout=True)


RAGGED = [1, 7, 64, 65, 127, 128, 129, 300, 0, 263]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 37), (False, 0), (False, 50), (True, 1)])
def test_ragged_self_attention(d, causal, window):
    check(case(RAGGED, d=d, seed=d + window), causal, window, what="ragged", bounds=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 20)])
def test_ragged_cross_lengths(d, causal, window):
    lq = [200, 1, 0, 77, 130, 129, 5]
    lk = [64, 300, 5, 0, 1, 257, 140]
    check(case(lq, lk, H=3, d=d, seed=3 * d + window), causal, window, what="cross", bounds=True)


@pytest.mark.parametrize("lq,H", [([5], 1), ([130, 7, 300], 3), ([1000], 2), ([64] * 9 + [129], 1)])
@pytest.mark.parametrize("window", [37, 300])
def test_window_queues_few_items(lq, H, window):
    # Both passes pop from per-XCD queues under a window: few items, and item counts
    # that are not a multiple of eight, exercise empty queues and stealing.
    check(W.make_case(lq, None, H=H, d=128, dtype=W.BF16, seed=sum(lq) + H + window, with_dout=True), True,
          window, what=f"queues {len(lq)} seqs", bounds=True)


def test_workload5_bwd_every_pair():
    # The whole sliding-window batch (its longest sequences included), every
    # (sequence, head) pair of dQ, dK and dV. With fp32 gradients every element is
    # held to 2e-2. With bf16 gradients (what a bf16 training step stores) the few
    # elements above 2e-2 must be rounding-limited and within their rounding bound:
    # a gradient of magnitude 4 to 8 is stored to within 2^-6 by bf16 itself.
    w = W.workload(5)
    say(f"[bwd] w5 B={w.B} H={w.H} Tq={w.q.shape[0]} causal={w.causal} window={w.window}")
    ro, rl, rq, rk, rv = oracle.bwd(w.q, w.k, w.v, w.dout, w.q_offsets, w.k_offsets, "softmax", w.causal, w.window,
                                    w.scale)
    for gdt, tag in ((torch.float32, "fp32 grads"), (torch.bfloat16, "bf16 grads")):
        dq, dk, dv = run_fwd_bwd(w, w.causal, w.window, grad_dtype=gdt)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            terms_at = None
            if gdt == torch.bfloat16:
                terms_at = (lambda idx, name=name:
                            softmax_grad_terms_at(w, w.causal, w.window, ro, rl, name, idx))
            st = compare(to_host64(got), ref, w.dtype, f"w5 bwd {name} ({tag})", terms_at=terms_at, report=True)
            say(f"      {name} {tag}: {st}")


def test_fp32_gradients_round_to_the_bf16_ones():
    # Same kernels, only the store differs: fp32 gradients rounded to bf16 (nearest
    # even) are bit for bit the bf16 gradients, for softmax and pointwise, with pair
    # splits (short key tiles) and every mask kind.
    for act, causal, window in (("softmax", True, 37), ("softmax", False, 0), ("silu", False, 0),
                                ("gelu", True, 0)):
        lq = [700, 300, 64, 1, 0, 129]
        lk = [64, 500, 64, 20, 3, 129]
        w = case(lq, lk, H=2, d=128, seed=91 + window)
        a = run_fwd_bwd(w, causal, window, act=act)
        b = run_fwd_bwd(w, causal, window, act=act, grad_dtype=torch.float32)
        for x, y in zip(a, b):
            assert y.dtype == torch.float32
            assert torch.equal(x.view(torch.int16), y.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("act", ["silu", "gelu"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (False, 50), (True, 37)])
def test_pointwise_ragged_self_attention(act, d, causal, window):
    check(case(RAGGED, d=d, seed=400 + d + window + (act == "gelu")), causal, window, what="ragged", act=act,
          bounds=True)


@pytest.mark.parametrize("act", ["silu", "gelu"])
@pytest.mark.parametrize("d", [64, 128])
def test_pointwise_cross_lengths(act, d):
    lq = [200, 1, 0, 77, 130, 129, 5]
    lk = [64, 300, 5, 0, 1, 257, 140]
    check(case(lq, lk, H=3, d=d, seed=500 + d), False, 0, what="cross", act=act, bounds=True)


@pytest.mark.parametrize("act,causal,window", [("softmax", False, 0), ("softmax", True, 0), ("softmax", True, 30),
                                               ("silu", False, 0), ("gelu", True, 0)])
def test_short_key_tiles_split_queries(act, causal, window):
    # Key tiles of at most 64 keys that visit two or more 64-query stages split the
    # stages' queries between two wave pairs and add their partial dK, dV: keys of
    # 64, 63, 1 and the last tiles of 129 and 192 keys, against 300-700 queries;
    # 65 and 128 keys (no split) and a one-stage tile (33 queries) beside them.
    lq = [700, 300, 450, 500, 640, 300, 512, 33]
    lk = [64, 63, 1, 129, 192, 65, 128, 40]
    check(case(lq, lk, H=2, d=128, seed=77 + window), causal, window, what="split-keys", act=act,
          bounds=True)


def test_workload3_silu_cross_bwd_every_pair():
    w = W.with_upstream_gradient(W.workload(3), 33)
    check(w, w.causal, w.window, what="w3 bwd", act=w.act, report=True)


def test_workload4_gelu_pooled_bwd_every_pair():
    w = W.with_upstream_gradient(W.workload(4), 44)
    check(w, w.causal, w.window, what="w4 bwd", act=w.act, report=True)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 100)])
def test_peaky_softmax_large_logits(causal, window):
    # Scale 0.5 at d = 128 (score standard deviation near 6): nearly one-hot weights. The
    # backward forms D_i = dO_i . O_i from the stored bf16 output, as the pages define it;
    # with one dominant key, dP_ij - D_i cancels to a small difference of two terms near
    # 10, so O's rounding (about sqrt(d) 2^-9 |O| in D_i) reaches dQ and dK at 1e-1 where
    # the gradients are near 18. Every element is held to its bf16 rounding bound plus
    # that derived term (stored_out_terms); dV, which does not use D, to its rounding
    # bound alone.
    w = case([300, 700, 64, 1], H=2, d=128, seed=79 + window)
    w.attn_scale = 0.5
    say(f"[bwd] peaky B={w.B} H={w.H} d={w.d} causal={causal} window={window} scale={w.scale}")
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    qo, ko = to_dev(w.q_offsets), to_dev(w.k_offsets)
    out, lse = ja.jagged_attn_fwd(q, k, v, qo, ko, causal=causal, window=window, scale=w.scale)
    dq, dk, dv = ja.jagged_attn_bwd(q, k, v, out, to_dev(w.dout), lse, qo, ko, causal=causal, window=window,
                                    scale=w.scale)
    torch.cuda.synchronize()
    ref_out, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", causal, window, w.scale)
    _, _, rq, rk, rv = oracle.bwd(w.q, w.k, w.v, w.dout, w.q_offsets, w.k_offsets, "softmax", causal, window,
                                  w.scale)
    _, tq, tk, tv = term_sums(w, "softmax", causal, window, grads=True)
    eq, ek = stored_out_terms(w, causal, window, to_host64(out), ref_out)
    for name, got, ref, terms, extra in (("dq", dq, rq, tq, eq), ("dk", dk, rk, tk, ek), ("dv", dv, rv, tv, 0.0)):
        err = np.abs(to_host64(got) - ref)
        lim = 2.0 ** -9 * (terms + np.abs(ref))
        tol = 2.0 * lim + 2e-3 + 1.01 * extra
        assert np.all(np.isfinite(err)), name
        worst = float(np.max(err / tol))
        say(f"      {name}: max abs {err.max():.3e} (|ref| up to {np.abs(ref).max():.1f}), mean abs {err.mean():.3e}, "
            f"max error / bound {worst:.3f}")
        assert worst <= 1.0, f"peaky {name}: error {worst:.3f} x its bound"
        assert err.mean() <= 2e-3 + float(np.mean(lim + extra)), f"peaky {name}: mean {err.mean():.3e}"


@pytest.mark.parametrize("H,d,window", [(16, 64, 0), (33, 32, 50), (12, 128, 200)])
def test_many_heads(H, d, window):
    # Head counts beyond the named workloads, odd ones included: row strides of H d
    # elements, per-head offsets, and work lists whose (sequence, head) items no longer
    # map onto the XCD-local queues one head per queue.
    w = case([130, 1, 0, 257, 64], H=H, d=d, seed=H + d)
    check_against_oracle(w, "softmax", True, window, what=f"H={H}", bounds=True)
    check(w, True, window, what=f"H={H}", bounds=True)


def test_identical_keys_give_zero_dq():
    w = case([150, 9, 300], d=64, seed=6)
    w.k[:] = w.k[0, 0]
    dq, _, _ = run_fwd_bwd(w, True, 40)
    assert torch.max(torch.abs(dq.float())).item() < 2e-2


def test_unseen_keys_get_zero_gradients():
    # causal, more keys than queries: keys at or past Lq are never seen
    w = case([100], [300], H=1, d=64, seed=7)
    _, dk, dv = run_fwd_bwd(w, True, 0)
    assert torch.count_nonzero(dk[100:]).item() == 0 and torch.count_nonzero(dv[100:]).item() == 0
    check(w, True, 0, what="unseen")


@pytest.mark.parametrize("act", ["softmax", "silu"])
def test_batch_without_keys(act):
    # Every sequence has queries but no keys (Tk = 0): out is 0 (lse -inf for softmax),
    # and so are the query gradients; there is no key gradient to write.
    w = case([5, 40, 0, 130], [0, 0, 0, 0], H=2, d=64, seed=12)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    qo, ko = to_dev(w.q_offsets), to_dev(w.k_offsets)
    out, lse = ja.jagged_attn_fwd(q, k, v, qo, ko, act=act, causal=True)
    torch.cuda.synchronize()
    assert k.shape[0] == 0 and torch.count_nonzero(out).item() == 0
    if act == "softmax":
        assert torch.isneginf(lse).all()
    dq, dk, dv = run_fwd_bwd(w, True, 0, act=act)
    assert torch.count_nonzero(dq).item() == 0 and dk.shape[0] == 0 and dv.shape[0] == 0


def test_batch_without_queries():
    # Sequences with keys but no queries (Tq = 0): nothing to compute or write; the key
    # gradients are zero.
    w = case([0, 0, 0], [7, 300, 0], H=2, d=128, seed=13)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    qo, ko = to_dev(w.q_offsets), to_dev(w.k_offsets)
    out, lse = ja.jagged_attn_fwd(q, k, v, qo, ko, causal=False)
    assert out.shape[0] == 0 and lse.shape[0] == 0
    dq, dk, dv = run_fwd_bwd(w, False, 0)
    assert dq.shape[0] == 0
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


def test_bitwise_determinism_and_permutation():
    lq = np.array([300, 0, 129, 64, 17, 700])
    w = case(lq, d=128, seed=8)
    a = run_fwd_bwd(w, True, 100)
    b = run_fwd_bwd(w, True, 100)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    perm = [3, 5, 0, 2, 1, 4]
    rows = np.concatenate([np.arange(w.q_offsets[i], w.q_offsets[i + 1]) for i in perm]).astype(np.int64)
    wp = W.Workload("perm", w.q[rows], w.k[rows], w.v[rows], W.offsets_from_lengths(lq[perm]),
                    W.offsets_from_lengths(lq[perm]), w.H, w.d, w.dtype, dout=w.dout[rows])
    c = run_fwd_bwd(wp, True, 100)
    idx = torch.from_numpy(rows).cuda()
    for x, y in zip(a, c):
        assert torch.equal(y.view(torch.int16), x.view(torch.int16)[idx])


def test_rejects_unsupported():
    w = case([10], d=64, seed=9)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    qo, ko = to_dev(w.q_offsets), to_dev(w.k_offsets)
    with pytest.raises(RuntimeError):  # softmax needs the forward's out and lse
        ja.jagged_attn_bwd(q, k, v, None, q, None, qo, ko, act="softmax")
    with pytest.raises(RuntimeError):  # the backward is bf16 only
        ja.jagged_attn_bwd(q.float(), k.float(), v.float(), None, q.float(), None, qo, ko, act="silu")
