"""GPU parity of the MXFP8 path ("Mixed Ultra-Low-Precision Training" section of
the GEM training post) against the fp64 oracle.

Quantizer: bit-exact E4M3 codes, E8M0 scales and scale offsets against the
oracle's quantizer (integer / byte work). Forward: the HIP kernel and the oracle
consume the same bytes (quantized by the oracle); the oracle rounds the softmax
weights exp(S - m) to E4M3 at scale 2^-8 from the final row max, the kernel from
its running max, so each weight of the two may differ by twice E4M3's rounding
(2^-3 of itself, or 2 * 2^-18 below the normal range). The derived per-element
bound is
    |out - ref| <= (2^-3 sum_j P_ij |V_j| + 2^-17 sum_j vis_ij |V_j|) / l_i
                   + 2^-8 |ref| + 2e-3
(P, l the unrounded softmax weights and their sum in fp64 on the dequantized
tensors; 2^-8 |ref| + 2e-3 for the bf16 output and fp32 accumulation), checked
element by element; lse (unaffected by the weight rounding) to 1e-3 relative.

Where the kernel's running max is the final row max from the start (rows whose
visible keys all lie in one 128-key stage: every row of a sequence of at most 128
keys, the first 128 rows of a causal sequence, window rows that do not straddle a
stage boundary), both sides round the same weights, and the tight bound applies:
    |out - ref| <= 2^-8 |ref| + 2e-3 + sum_{j ambiguous} step_j |V_j| / l_i
where a weight is ambiguous when 2^8 P_ij lies within 2^-12 of itself of an E4M3
rounding midpoint (fp32 scores in the kernel, fp64 in the oracle: either code is
a correct rounding there) and step_j is the E4M3 spacing at it, times 2^-8.
Cases: ragged lengths that are not multiples of 32 or 64, empty sequences,
causal, windowed, Lq != Lk, the MXFP8 workload on sampled (sequence, head)
pairs, and argument errors.
"""
import numpy as np
import pytest
import torch

import jagged_attention_recsys_amd as ja
import oracle
from jagged_attention_recsys_amd import workloads as W
from _parity import rows_of_pairs, say, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _dequant(x8, sc, soff, off):
    out = np.zeros(x8.shape, np.float64)
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    for b in range(len(off) - 1):
        for r in range(off[b], off[b + 1]):
            s = np.exp2(sc[soff[b] + (r - off[b]) // 32].astype(np.float64) - 127)  # [H, d/32]
            out[r] = dec[x8[r]] * np.repeat(s, 32, axis=1)
    return out


@pytest.mark.parametrize("d,H", [(128, 2), (64, 3), (32, 1)])
def test_quantizer_bit_exact(d, H):
    w = W.make_case([1, 31, 32, 33, 100, 0, 64, 300], H=H, d=d, dtype=W.BF16, seed=2000 + d)
    x = w.q.copy()
    x[40:45] = 0                     # zero rows inside a block
    x[133:165] = 0                   # a whole zero block
    x[200, 0, :] = W.f32_to_bf16_bits(np.full(d, 3.0e4, np.float32))  # large values
    x[201, 0, :5] = W.f32_to_bf16_bits(np.full(5, 1.0e-38, np.float32))  # subnormal-range values
    say(f"[mx quant] d={d} H={H} T={x.shape[0]}")
    r8, rsc, rsoff = oracle.mxfp8_quantize(x, w.q_offsets)
    g8, gsc, gsoff = ja.mxfp8_quantize(to_dev(x), to_dev(w.q_offsets))
    torch.cuda.synchronize()
    gsoff = gsoff.cpu().numpy()
    np.testing.assert_array_equal(gsoff, rsoff)
    np.testing.assert_array_equal(g8.cpu().numpy(), r8)
    np.testing.assert_array_equal(gsc.cpu().numpy()[:rsoff[-1]], rsc)


def _quantized(w):
    q = oracle.mxfp8_quantize(w.q, w.q_offsets)
    k = oracle.mxfp8_quantize(w.k, w.k_offsets)
    v = oracle.mxfp8_quantize(w.v, w.k_offsets)
    return q, k, v


def _scale_rows(sc, T, B):
    """The oracle's scales ([NB, H, d/32], NB = the blocks used) padded with zero rows
    to ceil(T/32) + B, the size the binding requires (what the quantizer allocates)."""
    n = max((T + 31) // 32 + B, 1)
    out = np.zeros((n,) + sc.shape[1:], dtype=np.uint8)
    out[:sc.shape[0]] = sc
    return out


def run_mx(w, q, k, v, causal, window):
    dev = lambda t: torch.from_numpy(np.ascontiguousarray(t)).cuda()
    Tq, Tk, B = w.q.shape[0], w.k.shape[0], w.B
    qs, ks, vs = _scale_rows(q[1], Tq, B), _scale_rows(k[1], Tk, B), _scale_rows(v[1], Tk, B)
    out, lse = ja.jagged_attn_fwd_mxfp8(dev(q[0]), dev(qs), dev(q[2]), dev(k[0]), dev(ks), dev(k[2]),
                                        dev(v[0]), dev(vs), to_dev(w.q_offsets), to_dev(w.k_offsets),
                                        causal=causal, window=window, scale=w.scale)
    torch.cuda.synchronize()
    return to_host64(out), to_host64(lse)


def _e4m3_grid():
    """Sorted non-negative finite E4M3 values (codes 0x00..0x7E)."""
    return np.sort(oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))


def _ambiguous_steps(x, grid):
    """For values x >= 0 (fp64) to be rounded to E4M3: the E4M3 spacing where x lies
    within 2^-12 x of a rounding midpoint, else 0."""
    i = np.clip(np.searchsorted(grid, x, side="right") - 1, 0, grid.size - 2)
    lo, hi = grid[i], grid[i + 1]
    mid = 0.5 * (lo + hi)
    return np.where(np.abs(x - mid) <= 2.0 ** -12 * x, hi - lo, 0.0)


def check(w, causal, window, pair_mask=None, what="", tight=False):
    """tight: rows whose visible keys lie in one 128-key stage are held to the tight
    bound (module docstring), every other row to the derived general bound."""
    say(f"[mx fwd] {what} B={w.B} H={w.H} Tq={w.q.shape[0]} Tk={w.k.shape[0]} causal={causal} window={window}")
    q, k, v = _quantized(w)
    out, lse = run_mx(w, q, k, v, causal, window)
    ref, rlse = oracle.fwd_mxfp8(q[0], q[1], q[2], k[0], k[1], k[2], v[0], v[1], w.q_offsets, w.k_offsets,
                                 causal, window, w.scale, pquant=True, pair_mask=pair_mask)
    qd = _dequant(*q, w.q_offsets)
    kd = _dequant(*k, w.k_offsets)
    vd = _dequant(*v, w.k_offsets)
    worst, n, esum, n_amb, n_tight = 0.0, 0, 0.0, 0, 0
    grid = _e4m3_grid()
    for b in range(w.B):
        q0, q1 = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        k0, k1 = int(w.k_offsets[b]), int(w.k_offsets[b + 1])
        if q1 == q0:
            continue
        i = np.arange(q1 - q0)[:, None]
        j = np.arange(k1 - k0)[None, :]
        vis = np.ones((q1 - q0, k1 - k0), dtype=bool)
        if causal:
            vis &= j <= i
        if window > 0:
            vis &= (i - j if causal else np.abs(i - j)) < window
        for h in range(w.H):
            if pair_mask is not None and not pair_mask[b, h]:
                continue
            if k1 == k0 or not vis.any():
                assert np.all(out[q0:q1, h] == 0)
                continue
            s = w.scale * qd[q0:q1, h] @ kd[k0:k1, h].T
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.where(vis, np.exp(s - np.where(np.isfinite(m), m, 0)), 0.0)
            l = p.sum(axis=1, keepdims=True)
            lsafe = np.where(l > 0, l, 1)
            av = np.abs(vd[k0:k1, h])
            r, g = ref[q0:q1, h], out[q0:q1, h]
            bound = (2.0 ** -3 * p @ av + 2.0 ** -17 * vis @ av) / lsafe
            tol = bound + 2.0 ** -8 * np.abs(r) + 2e-3
            if tight:
                # rows whose first and last visible key share a 128-key stage
                first = np.argmax(vis, axis=1)
                last = vis.shape[1] - 1 - np.argmax(vis[:, ::-1], axis=1)
                one = vis.any(axis=1) & (first // 128 == last // 128)
                steps = _ambiguous_steps(256.0 * p, grid) * vis
                n_amb += int(np.count_nonzero(steps[one]))
                n_tight += int(one.sum())
                tight_tol = 2.0 ** -8 * np.abs(r) + 2e-3 + (steps / 256.0) @ av / lsafe
                tol = np.where(one[:, None], tight_tol, tol)
            err = np.abs(g - r)
            assert np.all(np.isfinite(g)), what
            assert np.all(err <= tol), f"{what} b={b} h={h}: max excess {np.max(err - tol):.3e}"
            worst = max(worst, float(err.max()))
            esum += float(err.sum())
            n += err.size
            rows = vis.any(axis=1)
            gl, rl = lse[q0:q1, h][rows], rlse[q0:q1, h][rows]
            assert np.all(np.abs(gl - rl) <= 1e-3 * np.maximum(1.0, np.abs(rl))), f"{what} lse"
    say(f"      ok max_abs={worst:.3e} mean_abs={esum / max(n, 1):.3e} tight rows={n_tight} "
        f"ambiguous weights={n_amb}")
    if tight:
        assert n_tight > 0


RAGGED = [1, 7, 64, 65, 127, 128, 129, 300, 0, 263]


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 37), (False, 50)])
def test_ragged_self_attention(causal, window):
    w = W.make_case(RAGGED, H=2, d=128, dtype=W.BF16, seed=2100 + window + causal)
    check(w, causal, window, what="ragged")


@pytest.mark.parametrize("causal", [False, True])
def test_cross_lengths(causal):
    lq = [200, 1, 0, 77, 130, 129, 5]
    lk = [64, 300, 5, 0, 1, 257, 140]
    w = W.make_case(lq, lk, H=3, d=128, dtype=W.BF16, seed=2200 + causal)
    check(w, causal, 0, what="cross")


def test_workload8_sampled():
    w = W.workload(8)
    rng = np.random.default_rng(8)
    mask = np.zeros((w.B, w.H), dtype=bool)
    mask[int(np.argmax(w.lq)), 0] = True
    mask[int(np.argmin(w.lq)), w.H - 1] = True
    while mask.sum() < 6:
        mask[int(rng.integers(w.B)), int(rng.integers(w.H))] = True
    check(w, w.causal, w.window, pair_mask=mask, what="w8")


@pytest.mark.parametrize("causal", [False, True])
def test_one_stage_keys_tight_bound(causal):
    # Every sequence's keys fit one 128-key stage, so the running max is the row max
    # from the start and both sides round the same weights.
    lq = [300, 1, 77, 513, 200, 129, 64]
    lk = [128, 1, 64, 100, 33, 127, 0]
    w = W.make_case(lq, lk, H=2, d=128, dtype=W.BF16, seed=2600 + causal)
    check(w, causal, 0, what="one-stage", tight=True)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 50), (False, 60)])
def test_single_stage_rows_tight_bound(causal, window):
    # Sequences of several 128-key stages: the rows whose visible keys all lie in one
    # stage (the first 128 causal rows; window rows that do not straddle a stage
    # boundary) are held to the tight bound.
    lengths = [700, 129, 1, 300, 257, 0, 450]
    w = W.make_case(lengths, H=2, d=128, dtype=W.BF16, seed=2700 + causal + window)
    check(w, causal, window, what="single-stage rows", tight=True)


def test_rejects_unsupported_head_dim():
    w = W.make_case([40], H=1, d=64, dtype=W.BF16, seed=2300)
    q, k, v = _quantized(w)
    with pytest.raises(RuntimeError):
        run_mx(w, q, k, v, False, 0)


def test_quantizer_many_sequences():
    # more sequences than the prefix kernel's threads: each thread takes several
    rng = np.random.default_rng(2400)
    lengths = rng.integers(0, 70, size=2600)
    w = W.make_case(lengths, H=2, d=64, dtype=W.BF16, seed=2401)
    say(f"[mx quant] B={w.B} T={w.q.shape[0]}")
    r8, rsc, rsoff = oracle.mxfp8_quantize(w.q, w.q_offsets)
    g8, gsc, gsoff = ja.mxfp8_quantize(to_dev(w.q), to_dev(w.q_offsets))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gsoff.cpu().numpy(), rsoff)
    np.testing.assert_array_equal(g8.cpu().numpy(), r8)
    np.testing.assert_array_equal(gsc.cpu().numpy()[:rsoff[-1]], rsc)


def test_many_short_sequences_fwd():
    rng = np.random.default_rng(2500)
    lengths = rng.integers(0, 90, size=400)
    w = W.make_case(lengths, H=2, d=128, dtype=W.BF16, seed=2501)
    check(w, True, 0, what="short")
