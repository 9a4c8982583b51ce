"""Seeded synthetic jagged-attention inputs.

This module only draws numbers: sequence lengths, offsets and iid N(0,1)
tensors, rounded to bf16 where a workload asks for it. It holds none of the
attention arithmetic, so both the HIP path (through its tests and benchmark) and
the fp64 oracle can be fed from the same bytes.

The eight workloads follow the shapes the engineering post "GEM Training: How Meta
Doubled the Efficiency of Its LLM-Scale Ads Foundation Model" describes in its
"Challenge 1" section (jagged user histories from hundreds to tens of thousands of
tokens; self-attention, cross-attention with long queries and short key/value,
pooled multi-head attention with short queries and long key/value) and in its
"BlockAttention" section (sliding window over long histories, then fixed 64-token
blocks that attend only within themselves), and the GDPA section's ALU-only GELU
on inputs bounded by QK-norm. The pages give no sizes; the sizes below are this
library's synthetic stand-ins for the production traffic they describe.

Recipe (one ``numpy.random.default_rng(seed)`` stream per workload, seed = its
number): lengths first, then Q, K, V and dO, each one ``standard_normal(float32)``
draw of shape [T, H, d] (drawn in row chunks, which consumes the stream exactly as
one call would), for QK-normed batches each Q and K row (token, head) divided by
its L2 norm, then round-to-nearest-even to bf16 for the bf16 workloads.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"
F64 = "f64"  # float32 draws widened to float64 (oracle-only cases)

_CHUNK_ROWS = 1 << 16


@dataclass
class Workload:
    """A jagged batch. Arrays are numpy; bf16 tensors are stored as their uint16 bit patterns."""

    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_offsets: np.ndarray  # int32 [B+1]
    k_offsets: np.ndarray  # int32 [B+1]
    H: int
    d: int
    dtype: str
    act: str = "softmax"
    causal: bool = False
    window: int = 0
    dout: np.ndarray | None = None
    block: int = 0  # > 0: block-diagonal mask of this many tokens (self-attention only)
    attn_scale: float = 0.0  # > 0: the scale applied to Q K^T; 0: 1/sqrt(d)
    extra: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.q_offsets.shape[0] - 1)

    @property
    def scale(self) -> float:
        return float(self.attn_scale) if self.attn_scale > 0 else float(1.0 / np.sqrt(self.d))

    @property
    def lq(self) -> np.ndarray:
        return np.diff(self.q_offsets.astype(np.int64))

    @property
    def lk(self) -> np.ndarray:
        return np.diff(self.k_offsets.astype(np.int64))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    if off[-1] > np.iinfo(np.int32).max:
        raise ValueError("total token count exceeds int32 offsets")
    return off.astype(np.int32)


def _normal(rng: np.random.Generator, T: int, H: int, d: int, dtype: str, unit_rows: bool = False) -> np.ndarray:
    """One [T,H,d] standard-normal float32 draw, converted chunk by chunk to bound memory.
    unit_rows: each (token, head) row scaled to unit L2 norm before rounding (the
    QK-norm stand-in); the draw itself is the same."""
    npdt = {BF16: np.uint16, F32: np.float32, F64: np.float64}[dtype]
    out = np.empty((T, H, d), dtype=npdt)
    for r0 in range(0, T, _CHUNK_ROWS):
        r1 = min(T, r0 + _CHUNK_ROWS)
        x = rng.standard_normal((r1 - r0, H, d), dtype=np.float32)
        if unit_rows:
            x = x / np.linalg.norm(x, axis=-1, keepdims=True)
        out[r0:r1] = f32_to_bf16_bits(x) if dtype == BF16 else x
    return out


def log_uniform_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    return np.rint(np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))).astype(np.int64)


def lognormal_lengths(rng: np.random.Generator, n: int, median: float, sigma: float, cap: int) -> np.ndarray:
    x = np.rint(np.exp(rng.normal(np.log(median), sigma, size=n)))
    return np.clip(x, 1, cap).astype(np.int64)


def make_case(lq, lk=None, H=1, d=32, dtype=BF16, seed=0, act="softmax", causal=False,
              window=0, with_dout=False, shared_q_rows: int | None = None, name="case",
              qk_norm: bool = False) -> Workload:
    """A generic seeded jagged batch with given per-sequence lengths.

    ``lk=None`` means self-attention (lk = lq). ``shared_q_rows=r`` draws one [r,H,d]
    query block and replicates it for every sequence (pooled attention seeds); then
    ``lq`` is ignored and every sequence has r query rows.
    """
    rng = np.random.default_rng(seed)
    lk_arr = np.asarray(lq if lk is None else lk, dtype=np.int64)
    if shared_q_rows is not None:
        lq_arr = np.full(lk_arr.shape[0], shared_q_rows, dtype=np.int64)
    else:
        lq_arr = np.asarray(lq, dtype=np.int64)
    return _build(rng, name, lq_arr, lk_arr, H, d, dtype, act, causal, window, with_dout, shared_q_rows, qk_norm)


def with_upstream_gradient(w: Workload, seed: int) -> Workload:
    """Give ``w`` a seeded upstream gradient dO of the queries' shape (the named
    workloads other than 5 draw none)."""
    w.dout = _normal(np.random.default_rng(seed), int(w.q.shape[0]), w.H, w.d, w.dtype)
    return w


def _build(rng, name, lq, lk, H, d, dtype, act, causal, window, with_dout, shared_q_rows, qk_norm=False):
    qo, ko = offsets_from_lengths(lq), offsets_from_lengths(lk)
    Tq, Tk = int(qo[-1]), int(ko[-1])
    if shared_q_rows is not None:
        seeds = _normal(rng, shared_q_rows, H, d, dtype, qk_norm)
        q = np.tile(seeds, (lq.shape[0], 1, 1)) if lq.shape[0] > 0 else seeds[:0].copy()
    else:
        q = _normal(rng, Tq, H, d, dtype, qk_norm)
    k = _normal(rng, Tk, H, d, dtype, qk_norm)
    v = _normal(rng, Tk, H, d, dtype)
    dout = _normal(rng, Tq, H, d, dtype) if with_dout else None
    return Workload(name=name, q=q, k=k, v=v, q_offsets=qo, k_offsets=ko, H=H, d=d, dtype=dtype,
                    act=act, causal=causal, window=window, dout=dout)


# --- the eight named workloads ------------------------------------------------

WORKLOADS = {
    1: "tiny jagged softmax self-attention fwd, fp32: B=4 lengths {7,33,64,129}, H=2, d=32 "
       "(second run: SiLU/Lk)",
    2: "jagged causal softmax self-attention fwd (JFA), bf16: B=64, lengths log-uniform [128,4096], "
       "H=4, d=128",
    3: "GDPA cross-attention fwd, SiLU/Lk, bf16: B=128, query lengths log-uniform [512,8192], Lk=64, "
       "H=4, d=128",
    4: "GDPA pooled multi-head attention fwd, GELU/Lk, bf16: B=256, 32 shared query seeds, key lengths "
       "log-uniform [1024,16384], H=8, d=64",
    5: "jagged sliding-window causal softmax self-attention fwd+bwd, bf16: B=32, lengths lognormal "
       "(median 2048, sigma 1, cap 32768), window 1024, H=8, d=128",
    6: "jagged block-diagonal causal softmax self-attention fwd+bwd (BlockAttention), bf16: B=32, "
       "lengths lognormal (median 2048, sigma 1, cap 32768), blocks of 64 tokens, H=8, d=128",
    7: "GDPA causal self-attention with the ALU-only GELU (order-6 Taylor), QK-normed (unit-norm) "
       "queries and keys, scale 1, fwd+bwd, bf16: B=64, lengths log-uniform [128,4096], H=4, d=128",
    8: "jagged causal softmax self-attention fwd on MXFP8 Q/K/V (E4M3, [32,32] block scales), the batch of "
       "workload 2: B=64, lengths log-uniform [128,4096], H=4, d=128",
}


def workload(n: int, act: str | None = None, seed: int | None = None) -> Workload:
    """Build workload ``n`` (1..8) from its seed (default: n; 8 reuses workload 2's batch)."""
    rng = np.random.default_rng(n if seed is None else seed)
    if n == 1:
        lq = np.array([7, 33, 64, 129], dtype=np.int64)
        w = _build(rng, "w1", lq, lq, 2, 32, F32, act or "softmax", False, 0, False, None)
    elif n == 2:
        lq = log_uniform_lengths(rng, 64, 128, 4096)
        w = _build(rng, "w2", lq, lq, 4, 128, BF16, act or "softmax", True, 0, False, None)
    elif n == 3:
        lq = log_uniform_lengths(rng, 128, 512, 8192)
        lk = np.full(128, 64, dtype=np.int64)
        w = _build(rng, "w3", lq, lk, 4, 128, BF16, act or "silu", False, 0, False, None)
    elif n == 4:
        lk = log_uniform_lengths(rng, 256, 1024, 16384)
        lq = np.full(256, 32, dtype=np.int64)
        w = _build(rng, "w4", lq, lk, 8, 64, BF16, act or "gelu", False, 0, False, 32)
    elif n == 5:
        lq = lognormal_lengths(rng, 32, 2048.0, 1.0, 32768)
        w = _build(rng, "w5", lq, lq, 8, 128, BF16, act or "softmax", True, 1024, True, None)
    elif n == 6:
        lq = lognormal_lengths(rng, 32, 2048.0, 1.0, 32768)
        w = _build(rng, "w6", lq, lq, 8, 128, BF16, act or "softmax", True, 0, True, None)
        w.block = 64
    elif n == 8:
        w = workload(2, act=act, seed=2 if seed is None else seed)
        w.name = "w8"
        w.extra["mxfp8"] = True
    elif n == 7:
        lq = log_uniform_lengths(rng, 64, 128, 4096)
        w = _build(rng, "w7", lq, lq, 4, 128, BF16, act or "gelu_taylor", True, 0, True, None, qk_norm=True)
        w.attn_scale = 1.0
    else:
        raise ValueError(f"unknown workload {n}")
    w.extra["description"] = WORKLOADS[n]
    return w
