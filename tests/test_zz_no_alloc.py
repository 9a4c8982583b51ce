"""The no-alloc forward (jagged_attn_fwd_noalloc, for callers that cannot allocate
device memory) against the workspace-taking jagged_attn_fwd, through the C ABI:
two calls in a row on one GPU, the second with a smaller batch (the fixed buffer
keeps the first call's contents), each compared bit for bit with jagged_attn_fwd on
the same inputs and element by element with the fp64 oracle at the strict bound;
then the first batch again, after the smaller one."""
import numpy as np
import pytest
import torch

import jagged_attention_recsys_amd as ja
import oracle
from jagged_attention_recsys_amd import workloads as W
from _parity import compare, say, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _run_both(w, act, causal, window):
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    qo, ko = to_dev(w.q_offsets), to_dev(w.k_offsets)
    Tq = q.shape[0]
    ref_out, ref_lse = ja.jagged_attn_fwd(q, k, v, qo, ko, act=act, causal=causal, window=window, scale=w.scale)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((Tq, w.H), float("nan"), dtype=torch.float32, device=q.device) if act == "softmax" else None
    ja.jagged_attn_fwd_noalloc(q, k, v, qo, ko, out, lse, act=act, causal=causal, window=window, scale=w.scale)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


@pytest.mark.parametrize("act,causal,window", [("softmax", True, 0), ("silu", False, 0), ("softmax", True, 50)])
def test_noalloc_matches_fwd_on_two_calls(act, causal, window):
    big = W.make_case([700, 1, 0, 300, 129, 2000, 64], H=2, d=128, dtype=W.BF16, seed=3100 + window)
    small = W.make_case([33, 5, 200], H=2, d=128, dtype=W.BF16, seed=3200 + window)
    for name, w in (("first", big), ("second, smaller", small), ("third, the first again", big)):
        say(f"[noalloc] {name}: B={w.B} Tq={w.q.shape[0]} act={act} causal={causal} window={window}")
        out, lse, ref_out, ref_lse = _run_both(w, act, causal, window)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), name
        if act == "softmax":
            assert torch.equal(lse, ref_lse), name
        want, _ = oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, act, causal, window, w.scale)
        compare(to_host64(out), want, w.dtype, f"noalloc {name}")


def test_noalloc_rejects_oversized_batch():
    q = torch.zeros((8, 1, 64), dtype=torch.bfloat16, device="cuda")
    off = torch.tensor([0, 8], dtype=torch.int32, device="cuda")
    # A batch whose work list would not fit: many (empty) sequences are enough.
    many = torch.zeros(3_000_001, dtype=torch.int32, device="cuda")
    many[-1] = 8
    with pytest.raises(RuntimeError, match="no-alloc"):
        ja.jagged_attn_fwd_noalloc(q, q, q, many, many, torch.empty_like(q))
    out, _ = ja.jagged_attn_fwd_noalloc(q, q, q, off, off, torch.empty_like(q))  # still usable afterwards
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
