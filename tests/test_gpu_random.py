"""Seeded random batches against the fp64 oracle: forward (bf16 and fp32) and backward
(bf16), with sequence counts, head counts, head dims, ragged lengths (empty sequences,
cross-attention with short or long keys, short queries), masks and activations drawn
per case. Each case is a fixed seed, so a failure names a reproducible batch; the
tolerances are those of the other parity tests (the strict bf16 bound, rounding-limited
elements held to their own bound), except that the mean bound adds the mean of the
elements' own rounding bounds (tests/_parity.py: gradients summed over hundreds of
terms, such as a handful of keys under many queries, round to bf16 with a mean error
near 2e-3 on their own)."""
import numpy as np
import pytest

from jagged_attention_recsys_amd import workloads as W
from test_gpu_block import check as check_block
from test_gpu_bwd import check as check_bwd
from test_gpu_fwd import check_against_oracle
from test_gpu_mxfp8 import check as check_mx

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 10))
    H = int(rng.integers(1, 5))
    d = int(rng.choice([32, 64, 128]))
    kind = rng.choice(["self", "cross_short_k", "cross_short_q", "cross"])

    def lengths(lo, hi):
        L = rng.integers(lo, hi, size=B)
        L[rng.random(B) < 0.15] = 0  # some empty sequences
        return L.astype(np.int64)

    if kind == "self":
        lq = lengths(1, 700)
        lk = None
    elif kind == "cross_short_k":
        lq, lk = lengths(1, 900), lengths(1, 80)
    elif kind == "cross_short_q":
        lq, lk = lengths(1, 40), lengths(1, 1500)
    else:
        lq, lk = lengths(1, 500), lengths(1, 500)
    act = str(rng.choice(["softmax", "softmax", "silu", "gelu"]))
    causal = bool(rng.random() < 0.5)
    window = int(rng.choice([0, 0, 1, 17, 64, 300]))
    return dict(lq=lq, lk=lk, H=H, d=d, act=act, causal=causal, window=window, kind=str(kind))


@pytest.mark.parametrize("seed", range(40))
def test_random_bf16_fwd_bwd(seed):
    c = draw(seed)
    w = W.make_case(c["lq"], c["lk"], H=c["H"], d=c["d"], dtype=W.BF16, seed=seed, with_dout=True)
    what = f"random {seed} {c['kind']}"
    check_against_oracle(w, c["act"], c["causal"], c["window"], what=what, bounds=True, mean_rounding=True)
    check_bwd(w, c["causal"], c["window"], what=what, act=c["act"], bounds=True, mean_rounding=True)


@pytest.mark.parametrize("seed", range(10))
def test_random_fp32_fwd(seed):
    c = draw(100 + seed)
    w = W.make_case(c["lq"], c["lk"], H=c["H"], d=c["d"], dtype=W.F32, seed=seed)
    check_against_oracle(w, c["act"], c["causal"], c["window"], what=f"random fp32 {seed} {c['kind']}")


@pytest.mark.parametrize("seed", range(12))
def test_random_block_attention(seed):
    # Block-diagonal attention (blocks of 1 to 256 tokens), forward and backward.
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 8))
    L = rng.integers(0, 600, size=B).astype(np.int64)
    block = int(rng.choice([1, 4, 16, 32, 64, 128, 256]))
    causal = bool(rng.random() < 0.5)
    d = int(rng.choice([32, 64, 128]))
    w = W.make_case(L, None, H=int(rng.integers(1, 4)), d=d, dtype=W.BF16, seed=seed, with_dout=True)
    check_block(w, block, causal, what=f"random block {seed} block={block}", mean_rounding=True)


@pytest.mark.parametrize("seed", range(10))
def test_random_mxfp8_fwd(seed):
    # MXFP8 forward (d = 128, softmax) on random ragged self and cross batches, held to
    # the derived bound of the MXFP8 tests.
    c = draw(300 + seed)
    w = W.make_case(c["lq"], c["lk"], H=c["H"], d=128, dtype=W.BF16, seed=seed)
    check_mx(w, c["causal"], c["window"], what=f"random mxfp8 {seed} {c['kind']}")
