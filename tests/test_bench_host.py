"""Host checks of the benchmark's useful-work count (no GPU).

bench.py reports useful TFLOP/s as 4 d H x (visible query-key pairs) per forward, so the
pair count is pinned here: against a brute-force count of the visibility rule (query i
sees key j iff j < Lk, causal => j <= i, window W > 0 => i - j < W when causal and
|i - j| < W otherwise, blocks of G tokens => i // G == j // G), and against the closed
forms for causal self-attention, L (L + 1) / 2, and causal with a window W <= L,
W (W + 1) / 2 + (L - W) W.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def brute_pairs(lq, lk, causal, window, block=0):
    total = 0
    for Lq, Lk in zip(lq, lk):
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        ok = np.ones((Lq, Lk), dtype=bool)
        if causal:
            ok &= j <= i
        if window > 0:
            ok &= (i - j < window) if causal else (np.abs(i - j) < window)
        if block > 0:
            ok &= (i // block) == (j // block)
        total += int(ok.sum())
    return total


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 7), (False, 5), (True, 1), (False, 1)])
def test_pairs_match_brute_force(causal, window):
    rng = np.random.default_rng(11 + window + causal)
    lq = rng.integers(0, 90, size=12)
    lq[:3] = [0, 1, 64]
    lk = lq.copy()
    assert bench.visible_pairs(lq, lk, causal, window) == brute_pairs(lq, lk, causal, window)
    lk2 = rng.integers(0, 90, size=12)  # cross-attention lengths
    assert bench.visible_pairs(lq, lk2, causal, window) == brute_pairs(lq, lk2, causal, window)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 4, 64])
def test_block_pairs_match_brute_force(causal, block):
    rng = np.random.default_rng(block)
    lq = rng.integers(0, 200, size=8)
    lq[0] = 0
    assert bench.visible_pairs(lq, lq, causal, 0, block) == brute_pairs(lq, lq, causal, 0, block)


def test_closed_forms():
    L = np.array([1, 2, 100, 4096])
    assert bench.visible_pairs(L, L, True, 0) == int(sum(l * (l + 1) // 2 for l in L))
    W = 37
    L = np.array([37, 38, 500, 2048])
    assert bench.visible_pairs(L, L, True, W) == int(sum(W * (W + 1) // 2 + (l - W) * W for l in L))
    assert bench.visible_pairs(L, L, False, 0) == int((L * L).sum())
