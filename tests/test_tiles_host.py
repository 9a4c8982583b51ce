"""Host build of the kernels' per-row visibility ranges (csrc/ja_tiles.h).

The forward and both backward passes mask an element by testing its index
against one range per lane (the keys a query row sees, or the queries that see a
key), and skip or mask whole blocks by asking whether a range misses or covers
them. This compiles the header with g++ and checks the ranges and both block
tests against the mask written out element by element from the library's reading
of the masks: query i sees key j iff j < Lk, causal => j <= i, window W > 0 =>
(causal ? i - j < W : |i - j| < W), and with blocks of 2^bsh tokens
i >> bsh == j >> bsh.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "jagged_attention_recsys_amd", "csrc")
NO_BLOCK = 31


def _rule(i, j, Lk, causal, window, bsh):
    i = np.asarray(i)
    j = np.asarray(j)
    diff = i - j
    ok = j < Lk
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= (diff if causal else np.abs(diff)) < window
    if bsh < NO_BLOCK:
        ok &= (i >> bsh) == (j >> bsh)
    return ok


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("tiles") / "tiles_check")
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(ROOT, "tests", "tiles_check.cpp"), "-o", exe], check=True)
    return exe


def test_visible_ranges_match_the_rule(checker):
    rng = np.random.default_rng(11)
    cases = []
    for _ in range(6000):
        Lq, Lk = int(rng.integers(0, 90)), int(rng.integers(0, 90))
        row = int(rng.integers(0, 100))
        causal = int(rng.integers(0, 2))
        window = int(rng.choice([0, 1, 2, 5, 17, 64, 1000]))
        bsh = int(rng.choice([0, 1, 3, 5, 6, NO_BLOCK]))
        x0, n = int(rng.integers(0, 100)), int(rng.choice([1, 2, 32, 64]))
        cases.append((row, Lq, Lk, causal, window, bsh, x0, n))
    # extremes: indices near 2^31, huge windows and blocks
    big = (1 << 31) - 2
    cases += [(big, big + 1, big + 1, c, w, b, big - 40, 32) for c in (0, 1) for w in (0, 1, (1 << 31) - 1)
              for b in (0, 30, NO_BLOCK)]
    text = "".join(" ".join(map(str, c)) + "\n" for c in cases)
    out = subprocess.run([checker], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
    xs = np.arange(0, 128)
    for c, line in zip(cases, out):
        row, Lq, Lk, causal, window, bsh, x0, n = c
        klo, kw, qlo, qw, misses, covers = map(int, line.split())
        assert klo >= 0 and kw >= 0 and qlo >= 0 and qw >= 0, (c, line)
        if row > 1000:  # extremes: check around the row only
            xs_c = np.arange(max(0, row - 70), min(row + 70, (1 << 31) - 1), dtype=np.int64)
        else:
            xs_c = xs
        keys_ok = _rule(row, xs_c, Lk, causal, window, bsh)
        assert np.array_equal((xs_c >= klo) & (xs_c < klo + kw), keys_ok), ("keys", c, line)
        q_ok = (xs_c < Lq) & _rule(xs_c, row, Lk, causal, window, bsh)
        assert np.array_equal((xs_c >= qlo) & (xs_c < qlo + qw), q_ok), ("queries", c, line)
        blk = _rule(row, np.arange(x0, x0 + n, dtype=np.int64), Lk, causal, window, bsh)
        assert misses == int(not blk.any()) and covers == int(blk.all()), ("block", c, line)
