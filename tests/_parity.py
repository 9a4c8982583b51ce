"""Helpers for GPU parity tests: upload seeded workloads, run the HIP path through
its C ABI binding, compare against the fp64 oracle with the stated tolerances.

Tolerances:
  * fp32 inputs: max|x - y| / max|y| <= 1e-5 over all compared elements;
  * bf16 in / fp32 accumulate (the default everywhere): |x - y| <= 2e-2 for every
    element and mean|x - y| <= 2e-3 over all compared elements. The named workloads
    at full size are held to exactly this.
  * rounding-limited elements, only where a test passes the term sums: a bf16 result
    y = sum_j w_j u_j whose weights w_j (softmax or pointwise weights, dS) are rounded
    to bf16 before the product, and which is itself rounded to bf16, carries up to
    2^-9 (sum_j |w_j u_j| + |y|) of rounding whatever the kernel does. Where that
    bound exceeds 1e-2 (half the absolute tolerance: rows with few visible keys, whose
    weights are of order one, or large gradient sums), the element is held to twice
    the bound plus 2e-3 instead of 2e-2; every other element stays at 2e-2.
  * the pointwise backward (gradients that are unnormalised sums over up to Lq
    terms) is also held to the rounding bound on every element (bounded=True).
  * the mean bound 2e-3 is the stated one for the named workloads. Random batches
    (mean_rounding=True) may hold gradients summed over hundreds of terms with
    weights of order one (a handful of keys under many queries), where rounding the
    exact result to bf16 alone costs a mean error near 2e-3; they are held to 2e-3
    plus the mean of their elements' rounding bounds 2^-9 (terms + |ref|).

Every comparison is recorded in STATS; the session summary (tests/conftest.py)
prints the ones a test marks with report=True (the named workloads at full size).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

F32_REL = 1e-5
BF16_MAX = 2e-2
BF16_MEAN = 2e-3
BF16_ULP = 2.0 ** -9   # relative rounding of one bf16 rounding step (half a unit in the last place)

STATS: list[dict] = []


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if arr.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rows_of_pairs(offsets: np.ndarray, H: int, pair_mask: np.ndarray | None):
    """Boolean [T, H] mask of the rows belonging to selected (b, h) pairs."""
    T = int(offsets[-1])
    sel = np.zeros((T, H), dtype=bool)
    B = offsets.shape[0] - 1
    for b in range(B):
        for h in range(H):
            if pair_mask is None or pair_mask[b, h]:
                sel[offsets[b]:offsets[b + 1], h] = True
    return sel


def _f64(a):
    if a.dtype == np.uint16:
        return (np.ascontiguousarray(a).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _visible(Lq, Lk, causal, window, block):
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    vis = np.ones((Lq, Lk), dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= (i - j if causal else np.abs(i - j)) < window
    if block > 0:
        vis &= (i // block) == (j // block)
    return vis


def term_sums(w, act, causal, window, block=0, pair_mask=None, grads=False):
    """Per output element, sum_j |w_j u_j| of the product that forms it, in fp64 (the
    scale of its bf16 rounding bound): out_i = sum_j P_ij V_j; dV_j = sum_i P_ij dO_i,
    dK_j = scale sum_i dS_ij Q_i, dQ_i = scale sum_j dS_ij K_j. Softmax: P = exp(S -
    lse), dS = P (dO V^T - D); SiLU / GELU: P = act(Z)/Lk, dS = act'(Z) dO V^T / Lk.
    Returns t_out, or (t_out, t_dq, t_dk, t_dv) with grads."""
    q, k, v = w.q, w.k, w.v
    t_out = np.zeros(q.shape, dtype=np.float64)
    if grads:
        t_dq = np.zeros(q.shape, dtype=np.float64)
        t_dk = np.zeros(k.shape, dtype=np.float64)
        t_dv = np.zeros(k.shape, dtype=np.float64)
    c = np.sqrt(2.0 / np.pi)
    for b in range(w.B):
        q0, q1 = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        k0, k1 = int(w.k_offsets[b]), int(w.k_offsets[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0 or Lk == 0 or (pair_mask is not None and not pair_mask[b].any()):
            continue
        vis = _visible(Lq, Lk, causal, window, block)
        for h in range(w.H):
            if pair_mask is not None and not pair_mask[b, h]:
                continue
            qb, kb, vb = _f64(q[q0:q1, h]), _f64(k[k0:k1, h]), _f64(v[k0:k1, h])
            z = w.scale * qb @ kb.T
            if act == "softmax":
                zm = np.where(vis, z, -np.inf)
                m = zm.max(axis=1, keepdims=True)
                p = np.where(vis, np.exp(zm - np.where(np.isfinite(m), m, 0.0)), 0.0)
                l = p.sum(axis=1, keepdims=True)
                p = p / np.where(l > 0, l, 1.0)
            else:
                if act == "silu":
                    sg = 1.0 / (1.0 + np.exp(-z))
                    a, da = z * sg, sg + z * sg * (1.0 - sg)
                elif act == "gelu_taylor":
                    k2, k4, k6 = c / 2, (c * 0.044715 - c ** 3 / 3) / 2, (2 * c ** 5 / 15 - c ** 3 * 0.044715) / 2
                    a = 0.5 * z + k2 * z ** 2 + k4 * z ** 4 + k6 * z ** 6
                    da = 0.5 + 2 * k2 * z + 4 * k4 * z ** 3 + 6 * k6 * z ** 5
                else:
                    t = np.tanh(c * (z + 0.044715 * z ** 3))
                    a = 0.5 * z * (1.0 + t)
                    da = 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3 * 0.044715 * z * z)
                p = np.where(vis, a / Lk, 0.0)
            t_out[q0:q1, h] = np.abs(p) @ np.abs(vb)
            if grads:
                dob = _f64(w.dout[q0:q1, h])
                dp = dob @ vb.T
                if act == "softmax":
                    D = (p * dp).sum(axis=1, keepdims=True)
                    ds = p * (dp - D)
                else:
                    ds = np.where(vis, da * dp / Lk, 0.0)
                t_dv[k0:k1, h] = np.abs(p).T @ np.abs(dob)
                t_dk[k0:k1, h] = w.scale * np.abs(ds).T @ np.abs(qb)
                t_dq[q0:q1, h] = w.scale * np.abs(ds) @ np.abs(kb)
    return (t_out, t_dq, t_dk, t_dv) if grads else t_out


def stored_out_terms(w, causal, window, got_out, ref_out):
    """Per gradient element, a bound on what the softmax backward's D_i = dO_i . O_i moves
    when O is the forward's stored output (bf16) rather than the exact one: with
    e_i = sum_c |dO_ic| |O_stored,ic - O_exact,ic|, dS_ij moves by at most P_ij e_i, so
    dQ_ic by scale e_i sum_j P_ij |K_jc| and dK_jc by scale sum_i P_ij e_i |Q_ic| (dV does
    not use D). got_out, ref_out: [Tq, H, d] fp64. Returns (ext_dq, ext_dk)."""
    ext_dq = np.zeros(w.q.shape, dtype=np.float64)
    ext_dk = np.zeros(w.k.shape, dtype=np.float64)
    for b in range(w.B):
        q0, q1 = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        k0, k1 = int(w.k_offsets[b]), int(w.k_offsets[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0 or Lk == 0:
            continue
        vis = _visible(Lq, Lk, causal, window, 0)
        for h in range(w.H):
            qb, kb = _f64(w.q[q0:q1, h]), _f64(w.k[k0:k1, h])
            zm = np.where(vis, w.scale * qb @ kb.T, -np.inf)
            m = zm.max(axis=1, keepdims=True)
            p = np.where(vis, np.exp(zm - np.where(np.isfinite(m), m, 0.0)), 0.0)
            l = p.sum(axis=1, keepdims=True)
            p = p / np.where(l > 0, l, 1.0)
            e = (np.abs(_f64(w.dout[q0:q1, h])) * np.abs(got_out[q0:q1, h] - ref_out[q0:q1, h])).sum(axis=1)
            ext_dq[q0:q1, h] = w.scale * e[:, None] * (p @ np.abs(kb))
            ext_dk[k0:k1, h] = w.scale * (p * e[:, None]).T @ np.abs(qb)
    return ext_dq, ext_dk


def _record(what, stats, report):
    stats = dict(stats)
    stats["what"] = what
    stats["report"] = bool(report)
    STATS.append(stats)


def compare(got: np.ndarray, ref: np.ndarray, dtype: str, what: str, sel: np.ndarray | None = None,
            terms: np.ndarray | None = None, bounded: bool = False, report: bool = False,
            terms_at=None, mean_rounding: bool = False) -> dict:
    """Assert the tolerance for `dtype` ("f32" or "bf16"); returns the error statistics.

    sel: [T, H] rows to compare (None: all). terms: per-element sum |w_j u_j| (term_sums);
    without it every bf16 element is held to 2e-2. With it, rounding-limited elements
    (2^-9 (terms + |ref|) > 1e-2) are held to their rounding bound instead, and with
    bounded=True every element is also held to it. terms_at: for batches too large for
    term_sums, a function returning the term sums of given [n, 3] element indices; it
    is asked only for the elements above 2e-2, each of which must then be
    rounding-limited and within its bound."""
    if sel is None:
        sel = np.ones(got.shape[:2], dtype=bool)
    g, r = got[sel].reshape(-1), ref[sel].reshape(-1)
    if g.size == 0:
        return {"n": 0}
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in the HIP output"
    err = np.abs(g - r)
    stats = {"n": int(g.size), "max_abs": float(err.max()), "mean_abs": float(err.mean()),
             "max_ref": float(np.abs(r).max())}
    if dtype == "f32":
        rel = stats["max_abs"] / max(stats["max_ref"], 1e-30)
        stats["rel"] = rel
        _record(what, stats, report)
        assert rel <= F32_REL, f"{what}: relative error {rel:.3e} > {F32_REL} ({stats})"
        return stats
    limited = np.zeros(g.size, dtype=bool)
    mean_tol = BF16_MEAN
    if terms is not None:
        lim = BF16_ULP * (terms[sel].reshape(-1) + np.abs(r))
        if mean_rounding:
            mean_tol = BF16_MEAN + float(lim.mean())
            stats["mean_tol"] = mean_tol
        limited = lim > 0.5 * BF16_MAX
        allowed = 2.0 * lim + 2e-3
        check = limited | bounded
        stats["rounding_limited"] = int(limited.sum())
        stats["max_err_over_bound"] = float(np.max(err[check] / allowed[check])) if check.any() else 0.0
    if terms_at is not None:
        over = np.argwhere((np.abs(got - ref) > BF16_MAX) & sel[..., None])
        stats["above_2e-2"] = int(over.shape[0])
        if over.shape[0]:
            t = terms_at(over)
            rv = np.abs(ref[tuple(over.T)])
            ev = np.abs(got[tuple(over.T)] - ref[tuple(over.T)])
            lim = BF16_ULP * (t + rv)
            stats["above_2e-2_rounding_limited"] = int((lim > 0.5 * BF16_MAX).sum())
            stats["max_err_over_bound"] = float(np.max(ev / (2.0 * lim + 2e-3)))
            if not (np.all(lim > 0.5 * BF16_MAX) and stats["max_err_over_bound"] <= 1.0):
                _record(what, stats, report)  # the summary shows the failing case too
            assert np.all(lim > 0.5 * BF16_MAX), f"{what}: an element above 2e-2 is not rounding-limited ({stats})"
            assert stats["max_err_over_bound"] <= 1.0, f"{what}: error exceeds the bf16 rounding bound ({stats})"
        stats["max_abs_strict"] = float(np.max(np.where(np.abs(got - ref) > BF16_MAX, 0.0, np.abs(got - ref))[sel]))
    else:
        stats["max_abs_strict"] = float(err[~limited].max()) if (~limited).any() else 0.0
    _record(what, stats, report)
    assert stats["max_abs_strict"] <= BF16_MAX, \
        f"{what}: max abs error {stats['max_abs_strict']:.4e} > {BF16_MAX} ({stats})"
    if terms is not None:
        assert stats["max_err_over_bound"] <= 1.0, f"{what}: error exceeds the bf16 rounding bound ({stats})"
    assert stats["mean_abs"] <= mean_tol, f"{what}: mean abs error {stats['mean_abs']:.4e} > {mean_tol:.4e}"
    return stats


def softmax_grad_terms_at(w, causal, window, ref_out, ref_lse, which, idx):
    """term_sums of single softmax-gradient elements (which: "dq", "dk" or "dv"; idx: [n, 3]
    (row, head, channel)), from the oracle's own O and lse: dV_jc = sum_i P_ij dO_ic,
    dK_jc = scale sum_i dS_ij Q_ic, dQ_ic = scale sum_j dS_ij K_jc, P_ij = exp(s_ij - lse_i),
    dS_ij = P_ij (dO_i . V_j - dO_i . O_i), over the visible (i, j) of the sequence."""
    out = np.zeros(idx.shape[0])
    qoff, koff = w.q_offsets, w.k_offsets
    for n, (r, h, c) in enumerate(idx):
        if which == "dq":
            b = int(np.searchsorted(qoff, r, side="right") - 1)
            i = r - qoff[b]
        else:
            b = int(np.searchsorted(koff, r, side="right") - 1)
            j = r - koff[b]
        q0, q1, k0, k1 = (int(x) for x in (qoff[b], qoff[b + 1], koff[b], koff[b + 1]))
        vis = _visible(q1 - q0, k1 - k0, causal, window, 0)
        rows = np.array([i]) if which == "dq" else np.nonzero(vis[:, j])[0]
        cols = np.nonzero(vis[i])[0] if which == "dq" else np.array([j])
        qb = _f64(w.q[q0 + rows, h])
        kb = _f64(w.k[k0 + cols, h])
        vb = _f64(w.v[k0 + cols, h])
        dob = _f64(w.dout[q0 + rows, h])
        p = np.exp(w.scale * qb @ kb.T - ref_lse[q0 + rows, h][:, None])
        if which == "dv":
            out[n] = float(p[:, 0] @ np.abs(dob[:, c]))
            continue
        D = (dob * ref_out[q0 + rows, h]).sum(axis=1, keepdims=True)
        ds = p * (dob @ vb.T - D)
        if which == "dk":
            out[n] = w.scale * float(np.abs(ds[:, 0]) @ np.abs(qb[:, c]))
        else:
            out[n] = w.scale * float(np.abs(ds[0]) @ np.abs(kb[:, c]))
    return out


def sample_pairs(w, n_pairs: int, seed: int = 0) -> np.ndarray:
    """Pick (b, h) pairs for the oracle: the longest sequence, the shortest, and random others."""
    rng = np.random.default_rng(seed)
    B, H = w.B, w.H
    mask = np.zeros((B, H), dtype=bool)
    cost = w.lq * np.maximum(w.lk, 1)
    mask[int(np.argmax(cost)), 0] = True
    mask[int(np.argmin(cost)), H - 1] = True
    while mask.sum() < min(n_pairs, B * H):
        mask[rng.integers(B), rng.integers(H)] = True
    return mask
