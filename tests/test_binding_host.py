"""Host-side argument checks of the Python binding: every tensor's dtype, exact
shape, contiguity and device is validated before anything reaches the C ABI, so a
caller's undersized or mismatched buffer becomes a ValueError instead of an
out-of-bounds GPU access. Runs without a GPU: shapes are checked before the
device, and correctly shaped CPU tensors are rejected for not being on the GPU."""
import pytest
import torch

import jagged_attention_recsys_amd as ja

BF = torch.bfloat16


def qkv(Tq=10, Tk=12, H=2, d=64, dtype=BF):
    return (torch.zeros(Tq, H, d, dtype=dtype), torch.zeros(Tk, H, d, dtype=dtype),
            torch.zeros(Tk, H, d, dtype=dtype))


def offs(*v):
    return torch.tensor(v, dtype=torch.int32)


QO, KO = offs(0, 4, 10), offs(0, 5, 12)


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_forward_shapes():
    q, k, v = qkv()
    raises("k must have shape", ja.jagged_attn_fwd, q, torch.zeros(12, 3, 64, dtype=BF), v, QO, KO)
    raises("v must have shape", ja.jagged_attn_fwd, q, k, torch.zeros(11, 2, 64, dtype=BF), QO, KO)
    raises("k must be torch.bfloat16", ja.jagged_attn_fwd, q, k.float(), v, QO, KO)
    raises("k_offsets must have shape", ja.jagged_attn_fwd, q, k, v, QO, offs(0, 12))
    raises("q_offsets must be torch.int32", ja.jagged_attn_fwd, q, k, v, QO.long(), KO)
    raises("out must have shape", ja.jagged_attn_fwd, q, k, v, QO, KO, out=torch.zeros(9, 2, 64, dtype=BF))
    raises("lse must have shape", ja.jagged_attn_fwd, q, k, v, QO, KO, lse=torch.zeros(10, 3))
    raises("lse must be torch.float32", ja.jagged_attn_fwd, q, k, v, QO, KO, lse=torch.zeros(10, 2, dtype=BF))
    raises("workspace has 1 bytes", ja.jagged_attn_fwd, q, k, v, QO, KO, workspace=torch.zeros(1, dtype=torch.uint8))
    raises("q must be contiguous", ja.jagged_attn_fwd, torch.zeros(10, 64, 2, dtype=BF).transpose(1, 2), k, v, QO, KO)
    raises("q must be a float32 or bfloat16", ja.jagged_attn_fwd, q.half(), k, v, QO, KO)
    raises("must be a GPU tensor", ja.jagged_attn_fwd, q, k, v, QO, KO)


def test_backward_shapes():
    q, k, v = qkv()
    o, do, lse = torch.zeros_like(q), torch.zeros_like(q), torch.zeros(10, 2)
    f = ja.jagged_attn_bwd
    raises("dout must have shape", f, q, k, v, o, torch.zeros(10, 2, 32, dtype=BF), lse, QO, KO)
    raises("out must have shape", f, q, k, v, torch.zeros(11, 2, 64, dtype=BF), do, lse, QO, KO)
    raises("lse must have shape", f, q, k, v, o, do, torch.zeros(10), QO, KO)
    raises("k must have shape", f, q, torch.zeros(12, 2, 32, dtype=BF), v, o, do, lse, QO, KO)
    raises("dq must have shape", f, q, k, v, o, do, lse, QO, KO, dq=torch.zeros(9, 2, 64, dtype=BF))
    raises("dk must have shape", f, q, k, v, o, do, lse, QO, KO, dk=torch.zeros(10, 2, 64, dtype=BF))
    raises("dv must be torch.bfloat16", f, q, k, v, o, do, lse, QO, KO, dv=torch.zeros(12, 2, 64))
    raises("k_offsets must have shape", f, q, k, v, o, do, lse, QO, offs(0, 1, 2, 12))
    raises("must be a GPU tensor", f, q, k, v, o, do, lse, QO, KO)


def test_block_shapes():
    q, k, v = qkv(10, 10)
    o = offs(0, 4, 10)
    raises("k must have shape", ja.jagged_block_attn_fwd, q, torch.zeros(12, 2, 64, dtype=BF), v, o, 64)
    raises("lse must have shape", ja.jagged_block_attn_fwd, q, k, v, o, 64, lse=torch.zeros(9, 2))
    raises("dout must have shape", ja.jagged_block_attn_bwd, q, k, v, None, torch.zeros(9, 2, 64, dtype=BF), None,
           o, 64)
    raises("dk must have shape", ja.jagged_block_attn_bwd, q, k, v, None, q, None, o, 64,
           dk=torch.zeros(10, 1, 64, dtype=BF))
    raises("must be a GPU tensor", ja.jagged_block_attn_fwd, q, k, v, o, 64)


def test_mxfp8_shapes():
    u8 = torch.uint8
    q8, k8, v8 = (torch.zeros(70, 2, 128, dtype=u8), torch.zeros(40, 2, 128, dtype=u8),
                  torch.zeros(40, 2, 128, dtype=u8))
    qo, ko = offs(0, 30, 70), offs(0, 33, 40)
    nbq, nbk = (70 + 31) // 32 + 2, (40 + 31) // 32 + 2
    qs, ks, vs = (torch.zeros(nbq, 2, 4, dtype=u8), torch.zeros(nbk, 2, 4, dtype=u8),
                  torch.zeros(nbk, 2, 4, dtype=u8))
    f = ja.jagged_attn_fwd_mxfp8
    raises(r"q_scales must be \[>= 5", f, q8, qs[:4], qo, k8, ks, ko, v8, vs, qo, ko)
    raises(r"v_scales must be \[>= 4, 2, 4\]", f, q8, qs, qo, k8, ks, ko, v8, vs[:, :, :2].contiguous(), qo, ko)
    raises("v8 must have shape", f, q8, qs, qo, k8, ks, ko, v8[:39], vs, qo, ko)
    raises("k_scale_offsets must have shape", f, q8, qs, qo, k8, ks, offs(0, 40), v8, vs, qo, ko)
    raises("must be a GPU tensor", f, q8, qs, qo, k8, ks, ko, v8, vs, qo, ko)
    raises("d must be a positive multiple of 32", ja.mxfp8_quantize, torch.zeros(5, 1, 48, dtype=BF), offs(0, 5))
    raises("x must be torch.bfloat16", ja.mxfp8_quantize, torch.zeros(5, 1, 64), offs(0, 5))


def test_outputs_must_not_alias():
    # A written buffer that shares memory with an input or another output is refused
    # before anything is launched (checked on CPU tensors, before the device check).
    q, k, v = qkv()
    o, do, lse = torch.zeros_like(q), torch.zeros_like(q), torch.zeros(10, 2)
    raises("out overlaps q", ja.jagged_attn_fwd, q, k, v, QO, KO, out=q)
    raises("dq overlaps q", ja.jagged_attn_bwd, q, k, v, o, do, lse, QO, KO, dq=q)
    dkv = torch.zeros_like(k)
    raises("dk overlaps dv", ja.jagged_attn_bwd, q, k, v, o, do, lse, QO, KO, dk=dkv, dv=dkv)
    raises("dv overlaps v", ja.jagged_attn_bwd, q, k, v, o, do, lse, QO, KO, dv=v)
    # a view into the middle of an input counts as well
    big = torch.zeros(12, 2, 64, dtype=BF)
    raises("out overlaps q", ja.jagged_attn_fwd, big[2:], k, v, QO, KO, out=big[:10])
    ob = offs(0, 4, 10)
    raises("dq overlaps dout", ja.jagged_block_attn_bwd, q, k[:10], v[:10], None, do, None, ob, 64, dq=do)
    raises("out overlaps k", ja.jagged_block_attn_fwd, q, k[:10], v[:10], ob, 64, out=k[:10])
    raises("out overlaps q", ja.jagged_attn_fwd_noalloc, q, k, v, QO, KO, q)
    # disjoint views of one buffer are fine (the device check comes next)
    raises("must be a GPU tensor", ja.jagged_attn_bwd, q, k, v, o, do, lse, QO, KO, dk=big[:12].clone(),
           dv=torch.zeros_like(v))
