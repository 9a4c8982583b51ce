"""Helpers for GPU parity tests: upload seeded workloads, run the HIP path through
its C ABI binding, compare against the fp64 oracle with the stated tolerances.

Tolerances:
  * fp32 inputs: max|x - y| / max|y| <= 1e-5 over all compared elements;
  * bf16 in / fp32 accumulate: max|x - y| <= 2e-2 and mean|x - y| <= 2e-3 (strict:
    used for the named workloads).
  * non-strict bf16 (edge cases whose outputs can be large, e.g. one or two keys per
    sequence under SiLU/GELU): |x - y| <= 2e-2 + 2^-8 |y| elementwise and the same mean
    bound. The relative term is the arithmetic's own floor: P is rounded to bf16 before
    the second product and the output is rounded to bf16, each within 2^-9 relative, so
    an output of magnitude 6 already carries up to 0.023 of rounding.
  * bounded bf16 (the pointwise backward, whose gradients are unnormalised sums
    over up to Lq terms): |x - y| <= 2^-8 (sum |term| + |y|) + 2e-3 elementwise, the
    rounding bound of compare_bounded, and the same mean bound.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

F32_REL = 1e-5
BF16_MAX = 2e-2
BF16_MEAN = 2e-3
BF16_REL = 2.0 ** -8


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


def compare(got: np.ndarray, ref: np.ndarray, dtype: str, what: str, sel: np.ndarray | None = None,
            strict: bool = True) -> dict:
    """Assert the tolerance for `dtype` ("f32" or "bf16"); returns the error statistics."""
    if sel is not None:
        got, ref = got[sel], ref[sel]
    got = got.reshape(-1)
    ref = ref.reshape(-1)
    if got.size == 0:
        return {"n": 0}
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in the HIP output"
    err = np.abs(got - ref)
    stats = {"n": int(got.size), "max_abs": float(err.max()), "mean_abs": float(err.mean()),
             "max_ref": float(np.abs(ref).max())}
    if dtype == "f32":
        rel = stats["max_abs"] / max(stats["max_ref"], 1e-30)
        stats["rel"] = rel
        assert rel <= F32_REL, f"{what}: relative error {rel:.3e} > {F32_REL} ({stats})"
    elif strict:
        assert stats["max_abs"] <= BF16_MAX, f"{what}: max abs error {stats['max_abs']:.4e} > {BF16_MAX} ({stats})"
        assert stats["mean_abs"] <= BF16_MEAN, f"{what}: mean abs error {stats['mean_abs']:.4e} > {BF16_MEAN}"
    else:
        excess = float(np.max(err - BF16_REL * np.abs(ref)))
        stats["excess"] = excess
        assert excess <= BF16_MAX, f"{what}: |err| - 2^-8|ref| reaches {excess:.4e} > {BF16_MAX} ({stats})"
        assert stats["mean_abs"] <= BF16_MEAN, f"{what}: mean abs error {stats['mean_abs']:.4e} > {BF16_MEAN}"
    return stats


def compare_bounded(got: np.ndarray, ref: np.ndarray, terms: np.ndarray, what: str,
                    sel: np.ndarray | None = None) -> dict:
    """bf16 check against a per-element rounding bound.

    For an output that is a sum of products whose one factor was rounded to bf16
    (within 2^-9 relative) and which is itself rounded to bf16, the error is at
    most 2^-9 (sum |term| + |result|) plus fp32 accumulation noise. `terms` holds
    sum |term| per element (fp64); the assertion allows twice the bound plus
    2e-3, and the usual mean bound.
    """
    if sel is not None:
        got, ref, terms = got[sel], ref[sel], terms[sel]
    got, ref, terms = got.reshape(-1), ref.reshape(-1), terms.reshape(-1)
    if got.size == 0:
        return {"n": 0}
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in the HIP output"
    err = np.abs(got - ref)
    allowed = BF16_REL * (terms + np.abs(ref)) + 2e-3
    ratio = float(np.max(err / allowed))
    stats = {"n": int(got.size), "max_abs": float(err.max()), "mean_abs": float(err.mean()),
             "max_ref": float(np.abs(ref).max()), "max_err_over_bound": ratio}
    assert ratio <= 1.0, f"{what}: error exceeds the rounding bound ({stats})"
    assert stats["mean_abs"] <= BF16_MEAN, f"{what}: mean abs error {stats['mean_abs']:.4e} > {BF16_MEAN}"
    return stats


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
