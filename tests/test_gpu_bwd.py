"""GPU parity of the jagged attention backward against the fp64 oracle.

Softmax: the HIP forward produces out and lse (as a training step would), the HIP
backward then produces dQ, dK and dV; the oracle computes all three from its own
fp64 forward. Pointwise SiLU / GELU: the backward reads neither out nor lse (both
are passed as None). Cases: ragged batches spanning several tiles with every
mask, d in {32, 64, 128}, asymmetric lengths, the full sliding-window workload
and the SiLU cross-attention and GELU pooled workloads on sampled (sequence,
head) pairs, a closed form (identical keys give dQ = 0), keys no query sees
(zero gradients), bitwise determinism and sequence-order invariance, and guard
bands around every gradient.
"""
import numpy as np
import pytest
import torch

import jagged_attention_recsys_amd as ja
import oracle
from jagged_attention_recsys_amd import workloads as W
from _parity import compare, compare_bounded, rows_of_pairs, say, to_dev, to_host64

pytestmark = pytest.mark.gpu

GUARD = 2


def guarded(shape, dtype):
    full = torch.full((shape[0] + 2 * GUARD,) + tuple(shape[1:]), float("nan"), dtype=dtype, device="cuda")
    return full, full[GUARD:GUARD + shape[0]]


def run_fwd_bwd(w, causal, window, dout=None, act="softmax"):
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    qo, ko = to_dev(w.q_offsets), to_dev(w.k_offsets)
    if act == "softmax":
        out, lse = ja.jagged_attn_fwd(q, k, v, qo, ko, act=act, causal=causal, window=window, scale=w.scale)
    else:
        out = lse = None  # the pointwise backward needs neither
    do = to_dev(w.dout if dout is None else dout)
    fq, dq = guarded(q.shape, q.dtype)
    fk, dk = guarded(k.shape, k.dtype)
    fv, dv = guarded(v.shape, v.dtype)
    ja.jagged_attn_bwd(q, k, v, out, do, lse, qo, ko, act=act, causal=causal, window=window, scale=w.scale,
                       dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for f, n in ((fq, q.shape[0]), (fk, k.shape[0]), (fv, v.shape[0])):
        assert torch.isnan(f[:GUARD].float()).all() and torch.isnan(f[GUARD + n:].float()).all(), "guard band"
    return dq, dk, dv


def _f64(a):
    return W.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def pointwise_term_sums(w, act, causal, window, pair_mask=None):
    """Per gradient element, the sum of |terms| of its bf16-operand product (the
    rounding bound's scale): dV_j = sum_i P_ij dO_i, dK_j = scale sum_i dS_ij Q_i,
    dQ_i = scale sum_j dS_ij K_j with P = act(Z)/Lk and dS = act'(Z) dP / Lk."""
    tq = np.zeros(w.q.shape, dtype=np.float64)
    tk = np.zeros(w.k.shape, dtype=np.float64)
    tv = np.zeros(w.k.shape, dtype=np.float64)
    for b in range(w.B):
        q0, q1 = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        k0, k1 = int(w.k_offsets[b]), int(w.k_offsets[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0 or Lk == 0:
            continue
        if pair_mask is not None and not pair_mask[b].any():
            continue
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        vis = np.ones((Lq, Lk), dtype=bool)
        if causal:
            vis &= j <= i
        if window > 0:
            vis &= np.abs(i - j) < window
        for h in range(w.H):
            if pair_mask is not None and not pair_mask[b, h]:
                continue
            qb, kb, vb, dob = (_f64(x[r0:r1, h]) for x, r0, r1 in
                               ((w.q, q0, q1), (w.k, k0, k1), (w.v, k0, k1), (w.dout, q0, q1)))
            z = w.scale * qb @ kb.T
            if act == "silu":
                sg = 1.0 / (1.0 + np.exp(-z))
                a, da = z * sg, sg + z * sg * (1.0 - sg)
            elif act == "gelu_taylor":  # only the scale of the terms matters here
                c = np.sqrt(2.0 / np.pi)
                k2, k4, k6 = c / 2, (c * 0.044715 - c ** 3 / 3) / 2, (2 * c ** 5 / 15 - c ** 3 * 0.044715) / 2
                a = 0.5 * z + k2 * z ** 2 + k4 * z ** 4 + k6 * z ** 6
                da = 0.5 + 2 * k2 * z + 4 * k4 * z ** 3 + 6 * k6 * z ** 5
            else:
                c = np.sqrt(2.0 / np.pi)
                t = np.tanh(c * (z + 0.044715 * z ** 3))
                a = 0.5 * z * (1.0 + t)
                da = 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3 * 0.044715 * z * z)
            p = np.where(vis, a / Lk, 0.0)
            ds = np.where(vis, da * (dob @ vb.T) / Lk, 0.0)
            tv[k0:k1, h] = np.abs(p).T @ np.abs(dob)
            tk[k0:k1, h] = w.scale * np.abs(ds).T @ np.abs(qb)
            tq[q0:q1, h] = w.scale * np.abs(ds) @ np.abs(kb)
    return tq, tk, tv


def check(w, causal, window, pair_mask=None, what="", strict=False, act="softmax"):
    say(f"[bwd] {what} act={act} B={w.B} H={w.H} d={w.d} Tq={w.q.shape[0]} Tk={w.k.shape[0]} causal={causal} "
        f"window={window}")
    dq, dk, dv = run_fwd_bwd(w, causal, window, act=act)
    _, _, rq, rk, rv = oracle.bwd(w.q, w.k, w.v, w.dout, w.q_offsets, w.k_offsets, act, causal, window,
                                  w.scale, pair_mask=pair_mask)
    selq = rows_of_pairs(w.q_offsets, w.H, pair_mask)
    selk = rows_of_pairs(w.k_offsets, w.H, pair_mask)
    stats = {}
    if act == "softmax":
        for name, got, ref, sel in (("dq", dq, rq, selq), ("dk", dk, rk, selk), ("dv", dv, rv, selk)):
            stats[name] = compare(to_host64(got), ref, w.dtype, f"{name} {what}", sel, strict=strict)
    else:
        tq, tk, tv = pointwise_term_sums(w, act, causal, window, pair_mask)
        for name, got, ref, terms, sel in (("dq", dq, rq, tq, selq), ("dk", dk, rk, tk, selk),
                                           ("dv", dv, rv, tv, selk)):
            stats[name] = compare_bounded(to_host64(got), ref, terms, f"{name} {what}", sel)
    say(f"      ok {stats}")


def case(lq, lk=None, H=2, d=64, seed=0):
    return W.make_case(lq, lk, H=H, d=d, dtype=W.BF16, seed=seed, with_dout=True)


RAGGED = [1, 7, 64, 65, 127, 128, 129, 300, 0, 263]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 37), (False, 0), (False, 50), (True, 1)])
def test_ragged_self_attention(d, causal, window):
    check(case(RAGGED, d=d, seed=d + window), causal, window, what="ragged")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 20)])
def test_ragged_cross_lengths(d, causal, window):
    lq = [200, 1, 0, 77, 130, 129, 5]
    lk = [64, 300, 5, 0, 1, 257, 140]
    check(case(lq, lk, H=3, d=d, seed=3 * d + window), causal, window, what="cross")


def _sample_w5(w, n=6, max_len=8192, seed=5):
    rng = np.random.default_rng(seed)
    mask = np.zeros((w.B, w.H), dtype=bool)
    ok = np.nonzero(w.lq <= max_len)[0]
    longest = ok[np.argmax(w.lq[ok])]
    mask[longest, 0] = True
    mask[int(np.argmin(w.lq)), w.H - 1] = True
    while mask.sum() < n:
        mask[int(rng.choice(ok)), int(rng.integers(w.H))] = True
    return mask


def test_workload5_fwd_bwd_sampled():
    w = W.workload(5)
    check(w, w.causal, w.window, pair_mask=_sample_w5(w), what="w5", strict=True)


@pytest.mark.parametrize("act", ["silu", "gelu"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (False, 50), (True, 37)])
def test_pointwise_ragged_self_attention(act, d, causal, window):
    check(case(RAGGED, d=d, seed=400 + d + window + (act == "gelu")), causal, window, what="ragged", act=act)


@pytest.mark.parametrize("act", ["silu", "gelu"])
@pytest.mark.parametrize("d", [64, 128])
def test_pointwise_cross_lengths(act, d):
    lq = [200, 1, 0, 77, 130, 129, 5]
    lk = [64, 300, 5, 0, 1, 257, 140]
    check(case(lq, lk, H=3, d=d, seed=500 + d), False, 0, what="cross", act=act)


@pytest.mark.parametrize("act,causal,window", [("softmax", False, 0), ("softmax", True, 0), ("softmax", True, 30),
                                               ("silu", False, 0), ("gelu", True, 0)])
def test_short_key_tiles_split_queries(act, causal, window):
    # Key tiles of at most 64 keys that visit two or more 64-query stages split the
    # stages' queries between two wave pairs and add their partial dK, dV: keys of
    # 64, 63, 1 and the last tiles of 129 and 192 keys, against 300-700 queries;
    # 65 and 128 keys (no split) and a one-stage tile (33 queries) beside them.
    lq = [700, 300, 450, 500, 640, 300, 512, 33]
    lk = [64, 63, 1, 129, 192, 65, 128, 40]
    check(case(lq, lk, H=2, d=128, seed=77 + window), causal, window, what="split-keys", act=act)


def _sample_pairs(w, n, seed):
    rng = np.random.default_rng(seed)
    mask = np.zeros((w.B, w.H), dtype=bool)
    mask[int(np.argmax(w.lq * np.maximum(w.lk, 1))), 0] = True
    mask[int(np.argmin(w.lq)), w.H - 1] = True
    while mask.sum() < n:
        mask[int(rng.integers(w.B)), int(rng.integers(w.H))] = True
    return mask


def test_workload3_silu_cross_bwd_sampled():
    w = W.with_upstream_gradient(W.workload(3), 33)
    check(w, w.causal, w.window, pair_mask=_sample_pairs(w, 6, 3), what="w3", strict=True, act=w.act)


def test_workload4_gelu_pooled_bwd_sampled():
    w = W.with_upstream_gradient(W.workload(4), 44)
    check(w, w.causal, w.window, pair_mask=_sample_pairs(w, 6, 4), what="w4", strict=True, act=w.act)


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
