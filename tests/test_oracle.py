"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself:
  * library routines on padded dense tensors: torch's scaled_dot_product_attention,
    logsumexp, silu, gelu(approximate="tanh") and autograd, all in float64 on the
    CPU -- the padded computation that jagged attention must reproduce without the
    padding ("Jagged Sequence Flash Attention" section of the GEM training post);
  * closed forms (identical keys give the mean of the visible values, zero queries
    give zero under the pointwise activations, constant values are reproduced, a
    single visible key returns its value);
  * invariants (permuting the sequences of a batch permutes the outputs, bitwise);
  * central finite differences of the backward;
  * brute-force enumeration for the reference work list.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from jagged_attention_recsys_amd import workloads as W


# --------------------------------------------------------------------------
# independent dense references (torch float64, padded)
# --------------------------------------------------------------------------

def _visible_mask(Lq, Lk, causal, window, block=0):
    """Boolean [Lq, Lk] visibility, written from the reading: causal means j <= i
    (top-left aligned); a window W keeps W keys including the query's own position;
    a block size G keeps keys of the query's own G-token block."""
    i = torch.arange(Lq).view(-1, 1)
    j = torch.arange(Lk).view(1, -1)
    m = torch.ones(Lq, Lk, dtype=torch.bool)
    if causal:
        m &= j <= i
    if window > 0:
        diff = (i - j) if causal else (i - j).abs()
        m &= diff < window
    if block > 0:
        m &= torch.div(i, block, rounding_mode="floor") == torch.div(j, block, rounding_mode="floor")
    return m


def _to_f64(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(W.bf16_bits_to_f32(x).astype(np.float64))
    return torch.from_numpy(np.asarray(x, dtype=np.float64))


def dense_reference(w: W.Workload, act="softmax", causal=False, window=0, need_grad=False, dout=None, block=0):
    """Per-sequence padded dense attention with torch library calls. Returns out, lse
    and (optionally) gradients of sum(dout * out) w.r.t. q, k, v."""
    q, k, v = _to_f64(w.q), _to_f64(w.k), _to_f64(w.v)
    if need_grad:
        q.requires_grad_(True); k.requires_grad_(True); v.requires_grad_(True)
    Hn, d = w.H, w.d
    scale = 1.0 / math.sqrt(d)
    pieces, lses = [], []
    for b in range(w.B):
        qo, q1 = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        ko, k1 = int(w.k_offsets[b]), int(w.k_offsets[b + 1])
        Lq, Lk = q1 - qo, k1 - ko
        qb = q[qo:q1].permute(1, 0, 2)  # [H, Lq, d]
        kb = k[ko:k1].permute(1, 0, 2)
        vb = v[ko:k1].permute(1, 0, 2)
        mask = _visible_mask(Lq, Lk, causal, window, block)  # [Lq, Lk]
        has = mask.any(dim=1) if Lk > 0 else torch.zeros(Lq, dtype=torch.bool)
        if Lq == 0:
            ob = qb * 0.0
            lb = torch.zeros(Hn, 0, dtype=torch.float64)
        elif act == "softmax":
            if not bool(has.any()):
                ob = qb * 0.0
                lb = torch.full((Hn, Lq), -math.inf, dtype=torch.float64)
            else:
                safe = mask | (~has).view(-1, 1)  # keep SDPA finite on empty rows
                ob = F.scaled_dot_product_attention(qb.unsqueeze(0), kb.unsqueeze(0), vb.unsqueeze(0),
                                                    attn_mask=safe, scale=scale)[0]
                ob = ob * has.view(1, -1, 1)
                s = scale * torch.matmul(qb, kb.transpose(1, 2))
                lb = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
        else:
            fn = F.silu if act == "silu" else (lambda x: F.gelu(x, approximate="tanh"))
            s = scale * torch.matmul(qb, kb.transpose(1, 2))
            p = fn(s) * mask
            ob = torch.matmul(p, vb) / (Lk if Lk > 0 else 1)
            lb = torch.full((Hn, Lq), math.nan, dtype=torch.float64)
        pieces.append(ob.permute(1, 0, 2))
        lses.append(lb.detach().permute(1, 0))
    outs = torch.cat(pieces, dim=0) if pieces else q * 0.0
    res = {"out": outs.detach().numpy().copy(),
           "lse": torch.cat(lses, dim=0).numpy() if lses else np.zeros((0, Hn))}
    if need_grad:
        dO = _to_f64(dout)
        (outs * dO).sum().backward()
        zero = lambda t: np.zeros(t.shape) if t.grad is None else t.grad.numpy()
        res.update(dq=zero(q), dk=zero(k), dv=zero(v))
    return res


def _rand_case(rng, dtype):
    B = int(rng.integers(1, 6))
    lq = rng.integers(0, 40, size=B)
    lq[rng.integers(0, B)] = int(rng.choice([0, 1, 39]))
    asym = bool(rng.integers(0, 2))
    lk = rng.integers(0, 40, size=B) if asym else lq
    H = int(rng.integers(1, 3))
    d = int(rng.choice([4, 8, 16]))
    return W.make_case(lq, lk, H=H, d=d, dtype=dtype, seed=int(rng.integers(1 << 30)))


def _relerr(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.size == 0:
        return 0.0
    denom = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / denom)


MASKS = [(False, 0), (True, 0), (True, 1), (True, 3), (False, 1), (False, 4), (True, 50)]


# --------------------------------------------------------------------------
# forward pins
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_softmax_matches_padded_sdpa(causal, window, dtype):
    rng = np.random.default_rng(100 + 7 * window + int(causal) + (dtype == W.BF16))
    for _ in range(4):
        w = _rand_case(rng, dtype)
        out, lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", causal, window)
        ref = dense_reference(w, "softmax", causal, window)
        assert _relerr(out, ref["out"]) <= 1e-12
        fin = np.isfinite(ref["lse"])
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.all(lse[~fin] == -np.inf)
        if fin.any():
            assert _relerr(lse[fin], ref["lse"][fin]) <= 1e-12


@pytest.mark.parametrize("act", ["silu", "gelu"])
@pytest.mark.parametrize("causal,window", MASKS)
def test_pointwise_matches_padded_dense(act, causal, window):
    rng = np.random.default_rng(200 + 7 * window + int(causal) + (act == "gelu"))
    for _ in range(4):
        w = _rand_case(rng, W.BF16)
        out, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, act, causal, window)
        ref = dense_reference(w, act, causal, window)
        assert _relerr(out, ref["out"]) <= 1e-12


def test_workload1_against_sdpa_and_silu():
    w = W.workload(1)
    out, lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax")
    ref = dense_reference(w, "softmax")
    assert _relerr(out, ref["out"]) <= 1e-13
    assert _relerr(lse, ref["lse"]) <= 1e-13
    out2, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "silu")
    ref2 = dense_reference(w, "silu")
    assert _relerr(out2, ref2["out"]) <= 1e-13


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3), (False, 2)])
def test_identical_keys_give_mean_of_visible_values(causal, window):
    lq = np.array([5, 1, 9, 0, 12])
    w = W.make_case(lq, H=2, d=8, dtype=W.F32, seed=3)
    w.k[:] = w.k[0, 0]  # the same key vector everywhere
    out, lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", causal, window)
    scale = 1.0 / math.sqrt(w.d)
    for b in range(w.B):
        qo, ko, L = w.q_offsets[b], w.k_offsets[b], lq[b]
        for i in range(L):
            js = [j for j in range(L)
                  if (not causal or j <= i) and (window == 0 or abs(i - j) < window)]
            for h in range(w.H):
                expect = np.mean(w.v[ko + np.array(js), h].astype(np.float64), axis=0)
                np.testing.assert_allclose(out[qo + i, h], expect, rtol=1e-13, atol=1e-14)
                qk = float(np.dot(w.q[qo + i, h].astype(np.float64), w.k[0, 0].astype(np.float64)))
                assert abs(lse[qo + i, h] - (scale * qk + math.log(len(js)))) <= 1e-12


def test_causal_trailing_window_mean():
    """Identical keys, causal, window 3: row i averages v[max(0,i-2)..i]."""
    L = 7
    w = W.make_case([L], H=1, d=4, dtype=W.F64, seed=9)
    w.k[:] = 1.0
    w.v[:, 0, 0] = np.arange(L, dtype=w.v.dtype)
    out, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", True, 3)
    expect = [np.mean(np.arange(max(0, i - 2), i + 1)) for i in range(L)]
    np.testing.assert_allclose(out[:, 0, 0], expect, rtol=1e-14)


@pytest.mark.parametrize("act", ["silu", "gelu"])
def test_zero_queries_give_zero_pointwise(act):
    w = W.make_case([3, 17, 0, 8], [5, 2, 4, 0], H=2, d=16, dtype=W.BF16, seed=4)
    w.q[:] = 0
    out, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, act)
    assert np.all(out == 0.0)


def test_zero_queries_softmax_uniform_mean():
    w = W.make_case([6, 11], [9, 4], H=1, d=8, dtype=W.F32, seed=5)
    w.q[:] = 0
    out, lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax")
    for b in range(w.B):
        ko, k1 = w.k_offsets[b], w.k_offsets[b + 1]
        mean = w.v[ko:k1].astype(np.float64).mean(axis=0)
        for i in range(w.q_offsets[b], w.q_offsets[b + 1]):
            np.testing.assert_allclose(out[i], mean, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(lse[i], math.log(k1 - ko), rtol=1e-14)


def test_constant_values_reproduced_and_single_key():
    w = W.make_case([10, 4], H=2, d=8, dtype=W.F32, seed=6)
    w.v[:] = 0.625
    out, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", True, 0)
    np.testing.assert_allclose(out, 0.625, rtol=1e-14)
    # window 1 (non-causal): only the key at the query's own position is visible
    w = W.make_case([10, 4], H=2, d=8, dtype=W.F32, seed=7)
    out, lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", False, 1)
    np.testing.assert_array_equal(out, w.v.astype(np.float64))
    # causal: the first row of each sequence sees only its first key
    out, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", True, 0)
    for b in range(w.B):
        np.testing.assert_array_equal(out[w.q_offsets[b]], w.v[w.k_offsets[b]].astype(np.float64))


@pytest.mark.parametrize("act", ["silu", "gelu"])
def test_rank_one_pointwise_closed_form(act):
    """Q_i = e1, K_j = x_j e1 gives s_ij = scale x_j; out = (1/Lk) sum_j act(scale x_j) V_j."""
    Lk, d = 13, 8
    w = W.make_case([5], [Lk], H=1, d=d, dtype=W.F32, seed=8)
    w.q[:] = 0
    w.q[:, 0, 0] = 1
    x = np.linspace(-4.0, 4.0, Lk).astype(np.float32)
    w.k[:] = 0
    w.k[:, 0, 0] = x
    out, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, act)
    s = torch.tensor(x.astype(np.float64) / math.sqrt(d))
    a = F.silu(s) if act == "silu" else F.gelu(s, approximate="tanh")
    expect = (a.numpy()[:, None] * w.v[:, 0].astype(np.float64)).sum(axis=0) / Lk
    for i in range(5):
        np.testing.assert_allclose(out[i, 0], expect, rtol=1e-13, atol=1e-15)


def test_gelu_tanh_close_to_erf_gelu():
    """The tanh form stays within 5e-4 of the erf form (a library routine) on [-6, 6]."""
    Lk, d = 49, 4
    w = W.make_case([1], [Lk], H=1, d=d, dtype=W.F64, seed=1)
    w.q[:] = 0
    w.q[0, 0, 0] = 1
    x = np.linspace(-12.0, 12.0, Lk)
    w.k[:] = 0
    w.k[:, 0, 0] = x
    w.v[:] = 0
    out = []
    for j in range(Lk):  # one-hot values pick out each activation
        w.v[:] = 0
        w.v[j, 0, 0] = Lk
        o, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "gelu")
        out.append(o[0, 0, 0])
    exact = F.gelu(torch.tensor(x / 2.0)).numpy()
    assert np.max(np.abs(np.array(out) - exact)) < 5e-4


def _act_values(act, s):
    """act(s_j) for scores s (len(s) <= 64) read back through the oracle: one query
    e1, keys s_j sqrt(d) e1 (so scale q.k_j = s_j), values Lk e_j."""
    s = np.asarray(s, dtype=np.float64)
    n, d = len(s), 64
    w = W.make_case([1], [n], H=1, d=d, dtype=W.F64, seed=2)
    w.q[:] = 0
    w.q[0, 0, 0] = 1
    w.k[:] = 0
    w.k[:, 0, 0] = s * math.sqrt(d)
    w.v[:] = 0
    w.v[np.arange(n), 0, np.arange(n)] = n
    out, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, act)
    return out[0, 0, :n]


def test_gelu_taylor_is_the_order_6_series_of_tanh_gelu():
    """The ALU-only GELU equals the Taylor series of the tanh form through x^6,
    derived here symbolically by a library (sympy), to rounding."""
    sympy = pytest.importorskip("sympy")
    x = sympy.symbols("x")
    c = sympy.sqrt(2 / sympy.pi)
    series = sympy.series(sympy.Rational(1, 2) * x * (1 + sympy.tanh(c * (x + sympy.Rational(44715, 10**6) * x**3))),
                          x, 0, 7).removeO()
    f = sympy.lambdify(x, series, "numpy")
    s = np.linspace(-2.0, 2.0, 41)
    got = _act_values("gelu_taylor", s)
    np.testing.assert_allclose(got, f(s), rtol=1e-13, atol=1e-15)


def test_gelu_taylor_error_is_order_8_and_bounded():
    """Against the library's tanh GELU: the error shrinks like x^8 near 0 (a wrong
    x^4 or x^6 coefficient would leave x^4 or x^6), and stays within 1.2e-3 on the
    QK-norm range |x| <= 1."""
    s = np.array([0.1, 0.2, -0.1, -0.2])
    err = np.abs(_act_values("gelu_taylor", s) - F.gelu(torch.tensor(s), approximate="tanh").numpy())
    for a, b in ((err[0], err[1]), (err[2], err[3])):
        assert 0.9 * 2.0 ** 8 <= b / a <= 1.1 * 2.0 ** 8
    s = np.linspace(-1.0, 1.0, 64)
    err = np.abs(_act_values("gelu_taylor", s) - F.gelu(torch.tensor(s), approximate="tanh").numpy())
    assert 1.0e-3 < err.max() <= 1.2e-3


@pytest.mark.parametrize("act,causal,window", [("softmax", False, 0), ("softmax", True, 5),
                                               ("silu", False, 0), ("gelu", True, 0)])
def test_sequence_permutation_is_bitwise_invariant(act, causal, window):
    lq = np.array([9, 0, 23, 4, 17])
    lk = np.array([12, 3, 23, 1, 17])
    w = W.make_case(lq, lk, H=2, d=16, dtype=W.BF16, seed=11)
    out, lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, act, causal, window)
    perm = [3, 0, 4, 2, 1]
    qo, ko = w.q_offsets, w.k_offsets
    qrows = np.concatenate([np.arange(qo[b], qo[b + 1]) for b in perm]).astype(np.int64)
    krows = np.concatenate([np.arange(ko[b], ko[b + 1]) for b in perm]).astype(np.int64)
    out2, lse2 = oracle.fwd(w.q[qrows], w.k[krows], w.v[krows], W.offsets_from_lengths(lq[perm]),
                            W.offsets_from_lengths(lk[perm]), act, causal, window)
    assert np.array_equal(out2, out[qrows])
    assert np.array_equal(lse2, lse[qrows], equal_nan=True)


def test_pair_mask_selects_pairs_and_threads_are_deterministic():
    w = W.make_case([20, 31, 5], H=3, d=8, dtype=W.BF16, seed=12)
    full, lfull = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", True, 0, nthreads=1)
    many, lmany = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", True, 0, nthreads=7)
    assert np.array_equal(full, many) and np.array_equal(lfull, lmany)
    mask = np.zeros((3, 3), dtype=bool)
    mask[1, 2] = True
    part, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", True, 0, pair_mask=mask)
    rows = slice(w.q_offsets[1], w.q_offsets[2])
    assert np.array_equal(part[rows, 2], full[rows, 2])
    assert np.isnan(part[rows, 1]).all() and np.isnan(part[: w.q_offsets[1]]).all()


def test_empty_rows_and_sequences():
    # Lq > Lk with a causal window: late rows see no key
    w = W.make_case([8], [3], H=1, d=4, dtype=W.F32, seed=13)
    out, lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", True, 2)
    # row i sees keys j in (i-2, i] and j < 3: rows 0..3 see something, rows 4.. see nothing
    assert np.all(np.isfinite(lse[:4])) and np.all(lse[4:] == -np.inf)
    assert np.all(out[4:] == 0.0)
    w = W.make_case([4, 3], [0, 2], H=1, d=4, dtype=W.F32, seed=14)
    out, lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "silu")
    assert np.all(out[:4] == 0.0)


def test_rejects_bad_offsets():
    w = W.make_case([3, 4], H=1, d=4, dtype=W.F32, seed=15)
    with pytest.raises(ValueError):
        oracle.fwd(w.q, w.k, w.v, np.array([0, 5, 4], np.int32), w.k_offsets)


# --------------------------------------------------------------------------
# backward pins
# --------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3), (False, 2)])
def test_backward_matches_autograd(act, causal, window):
    rng = np.random.default_rng(300 + window + 2 * int(causal))
    for _ in range(3):
        w = _rand_case(rng, W.BF16)
        dout = W.f32_to_bf16_bits(rng.standard_normal(w.q.shape).astype(np.float32))
        out, lse, dq, dk, dv = oracle.bwd(w.q, w.k, w.v, dout, w.q_offsets, w.k_offsets, act, causal, window)
        ref = dense_reference(w, act, causal, window, need_grad=True, dout=dout)
        assert _relerr(out, ref["out"]) <= 1e-12
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert _relerr(got, ref[name]) <= 1e-11, name


def _f(w, dout, act, causal, window, q, k, v):
    out, _ = oracle.fwd(q, k, v, w.q_offsets, w.k_offsets, act, causal, window, nthreads=1)
    return float(np.sum(out * dout))


@pytest.mark.parametrize("act,causal,window", [("softmax", True, 2), ("softmax", False, 0),
                                               ("silu", False, 0), ("gelu", True, 0), ("gelu_taylor", False, 0),
                                               ("gelu_taylor", True, 2)])
def test_backward_central_differences(act, causal, window):
    w = W.make_case([4, 3], [5, 3], H=1, d=4, dtype=W.F32, seed=21)
    q, k, v = (w.q.astype(np.float64), w.k.astype(np.float64), w.v.astype(np.float64))
    dout = np.random.default_rng(22).standard_normal(q.shape)
    _, _, dq, dk, dv = oracle.bwd(q, k, v, dout, w.q_offsets, w.k_offsets, act, causal, window)
    eps = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in itertools.product(*[range(n) for n in arr.shape]):
            saved = arr[idx]
            arr[idx] = saved + eps
            fp = _f(w, dout, act, causal, window, q, k, v)
            arr[idx] = saved - eps
            fm = _f(w, dout, act, causal, window, q, k, v)
            arr[idx] = saved
            num[idx] = (fp - fm) / (2 * eps)
        assert np.max(np.abs(num - grad)) <= 1e-7 * max(1.0, np.max(np.abs(grad))), name


def test_backward_identical_keys_closed_form():
    """Identical keys: softmax rows are uniform over the visible keys, so dQ = 0 and
    dV_j = sum over rows i that see j of dO_i / |J(i)|."""
    L, window = 9, 4
    w = W.make_case([L], H=1, d=8, dtype=W.F64, seed=23)
    w.k[:] = w.k[0]
    dout = np.random.default_rng(24).standard_normal(w.q.shape)
    _, _, dq, dk, dv = oracle.bwd(w.q, w.k, w.v, dout, w.q_offsets, w.k_offsets, "softmax", True, window)
    assert np.max(np.abs(dq)) <= 1e-13
    expect = np.zeros_like(dv)
    for i in range(L):
        js = list(range(max(0, i - window + 1), i + 1))
        for j in js:
            expect[j] += dout[i] / len(js)
    np.testing.assert_allclose(dv, expect, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# work list
# --------------------------------------------------------------------------

def _brute_items(row_off, col_off, BM, BN, causal, window, transposed, block=0):
    items = []
    for b in range(len(row_off) - 1):
        Lr, Lc = row_off[b + 1] - row_off[b], col_off[b + 1] - col_off[b]
        for t in range((Lr + BM - 1) // BM):
            rows = np.arange(t * BM, min(Lr, t * BM + BM))
            if transposed:  # rows are keys, columns are queries
                m = _visible_mask(Lc, Lr, causal, window, block).numpy()[:, rows].T
            else:
                m = _visible_mask(len(rows) + rows[0], Lc, causal, window, block).numpy()[rows]
            cols = np.nonzero(m.any(axis=0))[0] if m.size else np.array([], dtype=np.int64)
            tiles = set((cols // BN).tolist())
            items.append((b, t, len(tiles)))
    return items


@pytest.mark.parametrize("causal,window,transposed", [(False, 0, False), (True, 0, False), (True, 5, False),
                                                      (False, 3, False), (True, 5, True), (True, 0, True),
                                                      (False, 0, True)])
def test_tile_list_matches_brute_force(causal, window, transposed):
    rng = np.random.default_rng(31 + window)
    lr = rng.integers(0, 60, size=9)
    lc = lr if causal else rng.integers(0, 60, size=9)
    ro, co = W.offsets_from_lengths(lr), W.offsets_from_lengths(lc)
    BM, BN = 8, 4
    items, costs = oracle.tile_list(ro, co, BM, BN, causal, window, transposed)
    brute = _brute_items(ro, co, BM, BN, causal, window, transposed)
    assert sorted((int(b), int(t), int(c)) for (b, t), c in zip(items, costs)) == sorted(brute)
    keys = [(-c, b, t) for (b, t), c in zip(items.tolist(), costs.tolist())]
    assert keys == sorted(keys)


@pytest.mark.parametrize("causal,transposed", [(False, False), (True, False), (True, True), (False, True)])
def test_tile_list_block_matches_brute_force(causal, transposed):
    rng = np.random.default_rng(41 + causal + 2 * transposed)
    lr = rng.integers(0, 70, size=9)
    ro = W.offsets_from_lengths(lr)
    BM, BN, G = 8, 4, 12
    items, costs = oracle.tile_list(ro, ro, BM, BN, causal, 0, transposed, block=G)
    brute = _brute_items(ro, ro, BM, BN, causal, 0, transposed, block=G)
    assert sorted((int(b), int(t), int(c)) for (b, t), c in zip(items, costs)) == sorted(brute)


def test_tile_list_cap_orders_by_capped_cost():
    ro = W.offsets_from_lengths([64, 200, 130])
    items, costs = oracle.tile_list(ro, ro, 16, 8, False, 0, False, cap=10)
    capped = np.minimum(costs, 10)
    assert np.all(np.diff(capped) <= 0)
    assert sorted(items[:, 0].tolist()) == sorted([0] * 4 + [1] * 13 + [2] * 9)


# --------------------------------------------------------------------------
# generator
# --------------------------------------------------------------------------

def test_generator_is_deterministic_and_rounds_like_torch():
    a = W.workload(2)
    b = W.workload(2)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.q_offsets, b.q_offsets)
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0]  # ties round to even
    ours = W.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_shapes():
    w1 = W.workload(1)
    assert w1.q.shape == (233, 2, 32) and list(w1.lq) == [7, 33, 64, 129]
    w3 = W.workload(3)
    assert w3.B == 128 and np.all(w3.lk == 64) and w3.lq.min() >= 512 and w3.lq.max() <= 8192
    w5 = W.workload(5)
    assert w5.B == 32 and w5.lq.max() <= 32768 and w5.dout is not None and w5.window == 1024


# --------------------------------------------------------------------------
# block-diagonal attention ("BlockAttention" section)
# --------------------------------------------------------------------------

def _resplit(lengths, G):
    """Lengths of the same rows cut into consecutive G-token pieces per sequence."""
    out = []
    for L in lengths:
        L = int(L)
        out += [G] * (L // G) + ([L % G] if L % G else [])
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G", [8, 64])
def test_block_attention_is_attention_on_resplit_sequences(causal, G):
    # Each G-token block attends only to itself, so block attention over a batch is
    # plain attention over the batch cut into G-token sequences (same rows, same
    # key order): forward and backward must agree exactly.
    lengths = [0, 1, G - 1, G, G + 1, 3 * G + 5, 2 * G]
    w = W.make_case(lengths, H=2, d=16, dtype=W.F64, seed=70 + G + causal, with_dout=True)
    rs = W.offsets_from_lengths(_resplit(lengths, G))
    o1, l1 = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", causal, 0, block=G)
    o2, l2 = oracle.fwd(w.q, w.k, w.v, rs, rs, "softmax", causal, 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    g1 = oracle.bwd(w.q, w.k, w.v, w.dout, w.q_offsets, w.k_offsets, "softmax", causal, 0, block=G)
    g2 = oracle.bwd(w.q, w.k, w.v, w.dout, rs, rs, "softmax", causal, 0)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_block_attention_against_sdpa(causal):
    w = W.make_case([0, 1, 30, 64, 65, 150, 200], H=2, d=32, dtype=W.F64, seed=81 + causal)
    out, lse = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, "softmax", causal, 0, block=64)
    ref = dense_reference(w, "softmax", causal, 0, block=64)
    assert _relerr(out, ref["out"]) < 1e-12
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.max(np.abs(lse[fin] - ref["lse"][fin])) < 1e-12


def test_block_attention_gradients_against_autograd():
    w = W.make_case([5, 64, 100, 130], H=2, d=16, dtype=W.F64, seed=83, with_dout=True)
    _, _, dq, dk, dv = oracle.bwd(w.q, w.k, w.v, w.dout, w.q_offsets, w.k_offsets, "softmax", True, 0,
                                  block=64)
    ref = dense_reference(w, "softmax", True, 0, need_grad=True, dout=w.dout, block=64)
    for got, want in ((dq, ref["dq"]), (dk, ref["dk"]), (dv, ref["dv"])):
        assert _relerr(got, want) < 1e-10


# --------------------------------------------------------------------------
# MXFP8 pins
# --------------------------------------------------------------------------

def _torch_e4m3(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_codes_match_torch():
    """Every finite code decodes as torch's float8_e4m3fn does, and encoding (ties to
    even) agrees with torch's conversion on every code, every midpoint between
    neighbouring codes and random values in [-448, 448]."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    ref = torch.tensor(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(vals, ref)
    pos = np.sort(np.unique(np.abs(vals)))
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(5)
    xs = np.concatenate([vals, mids, -mids, rng.uniform(-448, 448, 2000), rng.uniform(-1e-2, 1e-2, 500)])
    np.testing.assert_array_equal(oracle.e4m3_encode(xs), _torch_e4m3(xs))


def _mx_reference(x, off):
    """Block scale exponent floor(log2 amax) - 8 (numpy frexp) and element rounding by
    torch's float8_e4m3fn conversion, block by block."""
    xf = W.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else np.asarray(x, np.float64)
    T, H, d = xf.shape
    x8 = np.zeros((T, H, d), np.uint8)
    scales = []
    for b in range(len(off) - 1):
        for r0 in range(off[b], off[b + 1], 32):
            r1 = min(r0 + 32, off[b + 1])
            blk = xf[r0:r1].reshape(r1 - r0, H, d // 32, 32)
            amax = np.abs(blk).max(axis=(0, 3))  # [H, d/32]
            _, ex = np.frexp(amax)
            e = np.where(amax > 0, np.clip(ex - 1 - 8, -127, 127), -127)
            scales.append((e + 127).astype(np.uint8))
            v = np.clip(blk / np.exp2(e)[None, :, :, None], -448, 448)
            x8[r0:r1] = _torch_e4m3(v).reshape(r1 - r0, H, d)
    return x8, np.array(scales, dtype=np.uint8).reshape(-1, H, d // 32)


def test_mxfp8_quantize_against_library_reference():
    w = W.make_case([1, 31, 32, 33, 100, 0, 64], H=3, d=64, dtype=W.BF16, seed=40)
    x = w.q.copy()
    x[5:7] = 0  # a block with zero rows and channels
    x8, sc, soff = oracle.mxfp8_quantize(x, w.q_offsets)
    rx8, rsc = _mx_reference(x, w.q_offsets)
    np.testing.assert_array_equal(x8, rx8)
    np.testing.assert_array_equal(sc, rsc)
    np.testing.assert_array_equal(soff, np.concatenate([[0], np.cumsum((w.lq + 31) // 32)]))


def test_mxfp8_quantize_closed_forms():
    off = np.array([0, 40], dtype=np.int32)
    x = np.zeros((40, 1, 32), dtype=np.float64)
    x[3, 0, 5] = 2.0 ** -3          # block 0: amax a power of two -> stored as 256 (code 0x78)
    x[7, 0, 9] = -2.0 ** -4
    x[35, 0, 0] = 3.0               # block 1: amax 3 = 1.5 * 2 -> exponent 1 - 8, stored 384
    x8, sc, soff = oracle.mxfp8_quantize(x, off)
    assert list(sc[:, 0, 0]) == [127 - 3 - 8, 127 + 1 - 8]
    assert x8[3, 0, 5] == 0x78 and x8[7, 0, 9] == 0xF0 and x8[35, 0, 0] == oracle.e4m3_encode([384.0])[0]
    assert np.count_nonzero(x8) == 3
    z8, zs, _ = oracle.mxfp8_quantize(np.zeros((5, 2, 32)), np.array([0, 5], np.int32))
    assert not z8.any() and not zs.any()  # all-zero blocks: scale byte 0, zero codes


def test_mxfp8_quantize_error_bound_and_sequence_independence():
    w = W.make_case([70, 33, 5], H=2, d=64, dtype=W.F32, seed=41)
    x8, sc, soff = oracle.mxfp8_quantize(w.q, w.q_offsets)
    deq = np.zeros_like(w.q, dtype=np.float64)
    for b in range(w.B):
        for r in range(w.q_offsets[b], w.q_offsets[b + 1]):
            blk = soff[b] + (r - w.q_offsets[b]) // 32
            deq[r] = oracle.e4m3_decode(x8[r]) * np.exp2(np.repeat(sc[blk].astype(np.float64) - 127, 32, axis=1))
    x = w.q.astype(np.float64)
    # each block's largest element lands in [256, 448] (values above 448 times the scale
    # saturate); the rest lose at most half a unit of E4M3's last place, 2^-4 relative,
    # or 2^-10 of the scale below the normal range
    for b in range(w.B):
        for blk in range(soff[b], soff[b + 1]):
            for h in range(w.H):
                for c in range(w.d // 32):
                    codes = x8[w.q_offsets[b] + 32 * (blk - soff[b]):, h, 32 * c:32 * c + 32][:32]
                    codes = codes[:max(0, min(32, w.q_offsets[b + 1] - w.q_offsets[b] - 32 * (blk - soff[b])))]
                    assert 256 <= np.abs(oracle.e4m3_decode(codes)).max() <= 448
    scale_of = np.zeros_like(x)
    for b in range(w.B):
        for r in range(w.q_offsets[b], w.q_offsets[b + 1]):
            scale_of[r] = np.exp2(np.repeat(sc[soff[b] + (r - w.q_offsets[b]) // 32].astype(np.float64) - 127, 32, axis=1))
    sat = np.abs(x) > 448 * scale_of  # the top of a block's range saturates at 448 (<= 1/8 of it)
    assert np.all(np.abs(deq[sat]) == 448 * scale_of[sat])
    assert np.all(np.abs(deq - x)[~sat] <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * scale_of)[~sat])
    # blocks restart at each sequence: quantizing one sequence alone gives the same codes
    s1, s2 = int(w.q_offsets[1]), int(w.q_offsets[2])
    a8, asc, _ = oracle.mxfp8_quantize(w.q[s1:s2], np.array([0, s2 - s1], np.int32))
    np.testing.assert_array_equal(a8, x8[s1:s2])
    np.testing.assert_array_equal(asc, sc[soff[1]:soff[2]])


def _mx_case(lq, lk, d=64, H=2, seed=0):
    w = W.make_case(lq, lk, H=H, d=d, dtype=W.BF16, seed=seed)
    q = oracle.mxfp8_quantize(w.q, w.q_offsets)
    k = oracle.mxfp8_quantize(w.k, w.k_offsets)
    v = oracle.mxfp8_quantize(w.v, w.k_offsets)
    return w, q, k, v


def _dequant(t, off):
    x8, sc, soff = t
    out = np.zeros(x8.shape, np.float64)
    for b in range(len(off) - 1):
        for r in range(off[b], off[b + 1]):
            out[r] = oracle.e4m3_decode(x8[r]) * np.exp2(np.repeat(sc[soff[b] + (r - off[b]) // 32].astype(np.float64) - 127, 32, axis=1))
    return out


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 9)])
def test_fwd_mxfp8_without_p_rounding_is_attention_on_dequantized_inputs(causal, window):
    w, q, k, v = _mx_case([37, 64, 1, 90], [37, 64, 1, 90], seed=42)
    out, lse = oracle.fwd_mxfp8(q[0], q[1], q[2], k[0], k[1], k[2], v[0], v[1], w.q_offsets, w.k_offsets,
                                causal, window, w.scale, pquant=False)
    qd, kd, vd = _dequant(q, w.q_offsets), _dequant(k, w.k_offsets), _dequant(v, w.k_offsets)
    ref, rlse = oracle.fwd(qd, kd, vd, w.q_offsets, w.k_offsets, "softmax", causal, window, w.scale)
    np.testing.assert_array_equal(out, ref)
    np.testing.assert_array_equal(lse, rlse)
    # and that is torch SDPA on the dequantized tensors
    wd = W.Workload("deq", qd, kd, vd, w.q_offsets, w.k_offsets, w.H, w.d, W.F64)
    dense = dense_reference(wd, "softmax", causal, window)
    assert _relerr(out, dense["out"]) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_mxfp8_p_rounding_within_its_bound(causal):
    """Rounding P (<= 1) to E4M3 at scale 2^-8 moves each weight by at most 2^-4 of
    itself (or 2^-18 absolute below the normal range): |dO_i| <= sum_j dP_ij |V_j| / l_i."""
    w, q, k, v = _mx_case([90, 33], [90, 70], seed=43)
    args = (q[0], q[1], q[2], k[0], k[1], k[2], v[0], v[1], w.q_offsets, w.k_offsets, causal, 0, w.scale)
    out, lse = oracle.fwd_mxfp8(*args, pquant=True)
    ref, rlse = oracle.fwd_mxfp8(*args, pquant=False)
    np.testing.assert_array_equal(lse, rlse)
    qd, kd, vd = _dequant(q, w.q_offsets), _dequant(k, w.k_offsets), _dequant(v, w.k_offsets)
    for b in range(w.B):
        q0, q1 = w.q_offsets[b], w.q_offsets[b + 1]
        k0, k1 = w.k_offsets[b], w.k_offsets[b + 1]
        for h in range(w.H):
            s = w.scale * qd[q0:q1, h] @ kd[k0:k1, h].T
            vis = np.ones_like(s, dtype=bool)
            if causal:
                vis &= np.arange(k1 - k0)[None, :] <= np.arange(q1 - q0)[:, None]
            s = np.where(vis, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            l = p.sum(axis=1, keepdims=True)
            bound = (np.maximum(2.0 ** -4 * p, 2.0 ** -18) * vis) @ np.abs(vd[k0:k1, h]) / l
            err = np.abs(out[q0:q1, h] - ref[q0:q1, h])
            assert np.all(err <= bound * (1 + 1e-12) + 1e-15)
            assert err.max() > 0  # the rounding does act


def test_fwd_mxfp8_exact_when_weights_are_representable():
    """Identical keys: every visible weight is exp(0) = 1, stored exactly (256 at scale
    2^-8), so rounding P changes nothing."""
    w, q, k, v = _mx_case([20, 45], [20, 45], seed=44)
    k8 = k[0].copy()
    k8[:] = k8[0]
    ks = k[1].copy()
    ks[:] = ks[0]
    args = (q[0], q[1], q[2], k8, ks, k[2], v[0], v[1], w.q_offsets, w.k_offsets, True, 0, w.scale)
    a, _ = oracle.fwd_mxfp8(*args, pquant=True)
    b, _ = oracle.fwd_mxfp8(*args, pquant=False)
    np.testing.assert_array_equal(a, b)
