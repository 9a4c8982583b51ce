"""Race check of the LDS stage pipelining (forward, dQ pass, dK/dV pass).

The library is also built with JA_SINGLE_STAGE=1 (libjagged_attn_single_stage.so):
there every K/V (Q/dO) stage goes through one LDS buffer, loaded and then consumed
between two workgroup barriers, with no load in flight while a stage is read. The
arithmetic is the same, so its outputs must equal the double-buffered build's bit
for bit; a missing wait or barrier around the prefetched stage would show as a
difference. Cases: every forward layout (standard, split for short queries,
chunked for short keys with streamed stages) and the backward's two passes
(including short key tiles that split their query stages), over ragged batches
with causal, window and cross-attention masks, and the full sliding-window batch.
"""
import os

import numpy as np
import pytest
import torch

import jagged_attention_recsys_amd as ja
from jagged_attention_recsys_amd import _lib, build
from jagged_attention_recsys_amd import workloads as W
from _parity import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def single():
    if not os.path.exists(build.LIB_SINGLE_STAGE):
        pytest.fail(f"{build.LIB_SINGLE_STAGE} is not built (run __graft_entry__.build())")
    return _lib.open_library(build.LIB_SINGLE_STAGE)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _fwd_bwd(w, act, causal, window, bwd):
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    qo, ko = to_dev(w.q_offsets), to_dev(w.k_offsets)
    out, lse = ja.jagged_attn_fwd(q, k, v, qo, ko, act=act, causal=causal, window=window, scale=w.scale)
    res = [out] + ([lse] if lse is not None else [])
    if bwd:
        res += list(ja.jagged_attn_bwd(q, k, v, out, to_dev(w.dout), lse, qo, ko, act=act, causal=causal,
                                       window=window, scale=w.scale))
    torch.cuda.synchronize()
    return res


def _same(single, w, act, causal, window, bwd, what):
    say(f"[race] {what} B={w.B} Tq={w.q.shape[0]} Tk={w.k.shape[0]} act={act} causal={causal} window={window}")
    a = _fwd_bwd(w, act, causal, window, bwd)
    with _lib.using(single):
        b = _fwd_bwd(w, act, causal, window, bwd)
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(_bits(x), _bits(y)), f"{what}: output {i} differs between the builds"


RAGGED = [1, 7, 64, 65, 127, 128, 129, 300, 0, 513, 2000]


@pytest.mark.parametrize("act,causal,window", [("softmax", True, 0), ("softmax", False, 50), ("silu", False, 0),
                                               ("gelu", True, 100)])
def test_standard_layout_fwd_bwd(single, act, causal, window):
    w = W.make_case(RAGGED, H=2, d=128, dtype=W.BF16, seed=4100 + window, with_dout=True)
    _same(single, w, act, causal, window, True, "standard")


@pytest.mark.parametrize("d", [64, 128])
def test_cross_and_short_key_tiles(single, d):
    lq = [700, 300, 450, 500, 640, 300, 512, 33, 1, 0]
    lk = [64, 63, 1, 129, 192, 65, 128, 40, 300, 5]
    w = W.make_case(lq, lk, H=2, d=d, dtype=W.BF16, seed=4200 + d, with_dout=True)
    for act, causal, window in (("softmax", True, 30), ("silu", False, 0)):
        _same(single, w, act, causal, window, True, f"cross d={d}")


def test_split_and_chunked_layouts(single):
    rng = np.random.default_rng(4300)
    lq = rng.integers(0, 41, size=40)
    lk = rng.integers(0, 900, size=40)
    w = W.make_case(lq, lk, H=2, d=128, dtype=W.BF16, seed=4301)
    assert ja.fwd_tile_shape(w.B, 128, w.q.shape[0], w.k.shape[0])[0] == 32
    _same(single, w, "softmax", False, 0, False, "split")
    lq = [1100, 1, 0, 512, 513, 640, 2049, 700]
    lk = [64, 5, 3, 0, 1, 64, 63, 300]
    w = W.make_case(lq, lk, H=2, d=128, dtype=W.BF16, seed=4302)
    assert ja.fwd_tile_shape(w.B, 128, w.q.shape[0], w.k.shape[0])[0] == 512
    _same(single, w, "silu", False, 0, False, "chunked")


def test_sliding_window_workload(single):
    w = W.workload(5)
    _same(single, w, "softmax", True, w.window, True, "w5")
