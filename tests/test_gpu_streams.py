"""Calls on caller-supplied streams: the binding allocates each call's workspace and
outputs on the stream its kernels run on, so two calls on two streams (each with its
own workspace) are independent of each other and of work on torch's current stream.
Results are compared bitwise with the same calls on the current stream (the kernels
are deterministic)."""
import numpy as np
import pytest
import torch

import jagged_attention_recsys_amd as ja
from jagged_attention_recsys_amd import workloads as W
from _parity import to_dev

pytestmark = pytest.mark.gpu


def _inputs(lengths, seed):
    w = W.make_case(lengths, H=4, d=128, dtype=W.BF16, seed=seed, with_dout=True)
    return w, [to_dev(x) for x in (w.q, w.k, w.v, w.q_offsets, w.k_offsets, w.dout)]


def _fwd_bwd(t, stream=None):
    q, k, v, qo, ko, do = t
    out, lse = ja.jagged_attn_fwd(q, k, v, qo, ko, causal=True, window=300, stream=stream)
    dq, dk, dv = ja.jagged_attn_bwd(q, k, v, out, do, lse, qo, ko, causal=True, window=300, stream=stream)
    return out, lse, dq, dk, dv


def _same(a, b, what):
    for x, y, name in zip(a, b, ("out", "lse", "dq", "dk", "dv")):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), f"{what}: {name} differs"


def test_side_stream_matches_current_stream():
    _, t = _inputs([700, 1500, 1, 300], seed=3)
    ref = _fwd_bwd(t)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    got = _fwd_bwd(t, stream=s)
    s.synchronize()
    _same(got, ref, "side stream")


def test_two_streams_concurrently_with_work_on_the_current_stream():
    _, ta = _inputs([700, 1500, 1, 300], seed=3)
    _, tb = _inputs([2000, 64, 999], seed=4)
    ref_a, ref_b = _fwd_bwd(ta), _fwd_bwd(tb)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for s in (sa, sb):
        s.wait_stream(torch.cuda.current_stream())
    got_a = _fwd_bwd(ta, stream=sa)
    got_b = _fwd_bwd(tb, stream=sb)
    # Meanwhile the current stream allocates and overwrites fresh memory: blocks the
    # calls freed must not be among them while the calls' kernels still run.
    junk = [torch.full((1 << 22,), float(i), device="cuda") for i in range(16)]
    sa.synchronize()
    sb.synchronize()
    torch.cuda.synchronize()
    assert all(float(j[0]) == float(i) for i, j in enumerate(junk))
    _same(got_a, ref_a, "stream a")
    _same(got_b, ref_b, "stream b")


def test_schedule_on_side_stream():
    w, t = _inputs([700, 1500, 1, 300], seed=5)
    q, k, v, qo, ko, _ = t
    ref = ja.fwd_schedule(qo, ko, w.H, w.d, q.shape[0], k.shape[0], causal=True, window=300)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    got = ja.fwd_schedule(qo, ko, w.H, w.d, q.shape[0], k.shape[0], causal=True, window=300, stream=s)
    s.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())
