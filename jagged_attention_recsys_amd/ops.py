"""torch-facing binding of the C ABI: argument marshalling only.

Every step of the computation runs in the HIP library; torch only provides device
memory (outputs, workspace) and the current stream. Names mirror the C entry
points in include/jagged_attn.h.
"""
from __future__ import annotations

import functools
import inspect
import math

import torch

from . import _lib

ACT = {"softmax": 0, "silu": 1, "gelu": 2, "gelu_tanh": 2, "gelu_taylor": 3}
DTYPE = {torch.float32: 0, torch.bfloat16: 1}


def _act(act) -> int:
    if isinstance(act, str):
        if act not in ACT:
            raise ValueError(f"unknown activation {act!r}")
        return ACT[act]
    return int(act)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _on_stream(fn):
    """Run an entry point with `stream` (a torch.cuda.Stream, when given) as torch's
    current stream, so that the tensors it allocates (workspace, outputs) belong to
    the stream its kernels run on: freed on return, a workspace is not handed to other
    work on another stream while those kernels still use it, and any fill of such a
    tensor is ordered before them. Inputs produced on another stream are the caller's
    to order, as for any torch operation."""
    pos = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = args[pos] if len(args) > pos else kwargs.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)

    return wrapper


def _check(name: str, t, dtype=None, shape=None, dim=None, device=None) -> None:
    """Raise ValueError unless t is a contiguous tensor of the given dtype and exact
    shape (or number of dims) on `device`. Being on a GPU at all is checked last, by
    _on_gpu, so every shape check runs (and is tested) without a GPU."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _span(t):
    n = t.numel() * t.element_size()
    return (t.data_ptr(), t.data_ptr() + n) if n else None


def _disjoint(writes: dict, reads: dict) -> None:
    """Raise ValueError if a buffer the call writes shares memory with another buffer of
    the call (outputs may not alias inputs or each other: the backward's dK/dV pass,
    for one, reads Q and dO after its dQ pass has written dQ)."""
    w = [(n, _span(t)) for n, t in writes.items() if t is not None]
    r = [(n, _span(t)) for n, t in reads.items() if t is not None]
    for i, (n, a) in enumerate(w):
        for m, b in w[i + 1:] + r:
            if a and b and a[0] < b[1] and b[0] < a[1]:
                raise ValueError(f"{n} overlaps {m}: outputs must not share memory with inputs or other outputs")


def _on_gpu(name: str, t) -> None:
    """The last check before a launch: every other tensor is on t's device."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _check_offsets(name: str, t, n: int, device) -> None:
    _check(name, t, torch.int32, shape=(n,), device=device)


def _check_workspace(ws, need: int, device) -> None:
    if isinstance(ws, torch.Tensor) and ws.dtype == torch.uint8 and ws.dim() == 1 and ws.numel() < need:
        raise ValueError(f"workspace has {ws.numel()} bytes, the call needs {need}")
    _check("workspace", ws, torch.uint8, dim=1, device=device)


def fwd_workspace_size(B, H, d, Tq, Tk, act="softmax", causal=False, window=0, dtype=torch.bfloat16) -> int:
    return int(_lib.load().ja_fwd_workspace_size(B, H, d, Tq, Tk, _act(act), int(bool(causal)), int(window),
                                                 DTYPE[dtype]))


@_on_stream
def jagged_attn_fwd(q, k, v, q_offsets, k_offsets, act="softmax", causal=False, window=0, scale=None,
                    out=None, lse=None, workspace=None, stream=None):
    """Jagged attention forward. q: [Tq,H,d]; k, v: [Tk,H,d]; offsets: int32 [B+1] on the GPU.

    Returns (out [Tq,H,d], lse [Tq,H] float32 or None for pointwise activations).
    """
    lib = _lib.load()
    if not isinstance(q, torch.Tensor) or q.dtype not in DTYPE:
        raise ValueError(f"q must be a float32 or bfloat16 tensor")
    _check("q", q, dim=3)
    dtype, dev = q.dtype, q.device
    Tq, H, d = q.shape
    if not isinstance(k, torch.Tensor) or k.dim() != 3:
        raise ValueError("k must be a [Tk, H, d] tensor")
    Tk = k.shape[0]
    _check("k", k, dtype, shape=(Tk, H, d), device=dev)
    _check("v", v, dtype, shape=(Tk, H, d), device=dev)
    if not isinstance(q_offsets, torch.Tensor) or q_offsets.dim() != 1 or q_offsets.numel() < 1:
        raise ValueError("q_offsets must be an int32 [B+1] tensor")
    B = q_offsets.numel() - 1
    _check_offsets("q_offsets", q_offsets, B + 1, dev)
    _check_offsets("k_offsets", k_offsets, B + 1, dev)
    a = _act(act)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, dtype, shape=(Tq, H, d), device=dev)
    if a == 0 and lse is None:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
    elif a == 0:
        _check("lse", lse, torch.float32, shape=(Tq, H), device=dev)
    ws_bytes = int(lib.ja_fwd_workspace_size(B, H, d, Tq, Tk, a, int(bool(causal)), int(window), DTYPE[dtype]))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, ws_bytes, dev)
    _disjoint(dict(out=out, lse=lse, workspace=workspace),
              dict(q=q, k=k, v=v, q_offsets=q_offsets, k_offsets=k_offsets))
    _on_gpu("q", q)
    status = lib.jagged_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(k_offsets), B, H, d, Tq, Tk,
                                 a, int(bool(causal)), int(window), float(scale), DTYPE[dtype], _ptr(out),
                                 _ptr(lse) if a == 0 else None, _ptr(workspace), workspace.numel(),
                                 _stream(q.device, stream))
    _lib.check("jagged_attn_fwd", status)
    return out, (lse if a == 0 else None)


@_on_stream
def jagged_attn_fwd_noalloc(q, k, v, q_offsets, k_offsets, out, lse=None, act="softmax", causal=False, window=0,
                            scale=None, stream=None):
    """jagged_attn_fwd without a workspace: the library uses its fixed per-GPU device
    buffer (JA_NOALLOC_SCRATCH_BYTES), so neither this call nor the C entry point
    allocates anything. The caller passes the outputs: out [Tq,H,d] and, for softmax,
    lse [Tq,H] float32 (or None). Calls that overlap on one GPU share the buffer and
    race. Returns (out, lse)."""
    lib = _lib.load()
    if not isinstance(q, torch.Tensor) or q.dtype not in DTYPE:
        raise ValueError(f"q must be a float32 or bfloat16 tensor")
    _check("q", q, dim=3)
    dtype, dev = q.dtype, q.device
    Tq, H, d = q.shape
    if not isinstance(k, torch.Tensor) or k.dim() != 3:
        raise ValueError("k must be a [Tk, H, d] tensor")
    Tk = k.shape[0]
    _check("k", k, dtype, shape=(Tk, H, d), device=dev)
    _check("v", v, dtype, shape=(Tk, H, d), device=dev)
    if not isinstance(q_offsets, torch.Tensor) or q_offsets.dim() != 1 or q_offsets.numel() < 1:
        raise ValueError("q_offsets must be an int32 [B+1] tensor")
    B = q_offsets.numel() - 1
    _check_offsets("q_offsets", q_offsets, B + 1, dev)
    _check_offsets("k_offsets", k_offsets, B + 1, dev)
    _check("out", out, dtype, shape=(Tq, H, d), device=dev)
    a = _act(act)
    if lse is not None:
        _check("lse", lse, torch.float32, shape=(Tq, H), device=dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _disjoint(dict(out=out, lse=lse), dict(q=q, k=k, v=v, q_offsets=q_offsets, k_offsets=k_offsets))
    _on_gpu("q", q)
    status = lib.jagged_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(k_offsets), B, H, d, Tq,
                                         Tk, a, int(bool(causal)), int(window), float(scale), DTYPE[dtype],
                                         _ptr(out), _ptr(lse) if a == 0 else None, _stream(q.device, stream))
    _lib.check("jagged_attn_fwd_noalloc", status)
    return out, (lse if a == 0 else None)


def bwd_workspace_size(B, H, d, Tq, Tk, act="softmax", causal=False, window=0, dtype=torch.bfloat16) -> int:
    return int(_lib.load().ja_bwd_workspace_size(B, H, d, Tq, Tk, _act(act), int(bool(causal)), int(window),
                                                 DTYPE[dtype]))


@_on_stream
def jagged_attn_bwd(q, k, v, out, dout, lse, q_offsets, k_offsets, act="softmax", causal=False, window=0,
                    scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None, grad_dtype=None):
    """Backward of jagged_attn_fwd. Returns (dq, dk, dv), of q's dtype or of
    ``grad_dtype`` (torch.float32: the fp32 accumulators, unrounded).

    Softmax needs the forward's ``out`` and ``lse``; SiLU / GELU read neither
    (pass None)."""
    lib = _lib.load()
    if not isinstance(q, torch.Tensor) or q.dtype not in DTYPE:
        raise ValueError(f"q must be a float32 or bfloat16 tensor")
    _check("q", q, dim=3)
    dtype, dev = q.dtype, q.device
    Tq, H, d = q.shape
    if not isinstance(k, torch.Tensor) or k.dim() != 3:
        raise ValueError("k must be a [Tk, H, d] tensor")
    Tk = k.shape[0]
    _check("k", k, dtype, shape=(Tk, H, d), device=dev)
    _check("v", v, dtype, shape=(Tk, H, d), device=dev)
    _check("dout", dout, dtype, shape=(Tq, H, d), device=dev)
    # None passes through as a null pointer: the library rejects it for softmax.
    if out is not None:
        _check("out", out, dtype, shape=(Tq, H, d), device=dev)
    if lse is not None:
        _check("lse", lse, torch.float32, shape=(Tq, H), device=dev)
    if not isinstance(q_offsets, torch.Tensor) or q_offsets.dim() != 1 or q_offsets.numel() < 1:
        raise ValueError("q_offsets must be an int32 [B+1] tensor")
    B = q_offsets.numel() - 1
    _check_offsets("q_offsets", q_offsets, B + 1, dev)
    _check_offsets("k_offsets", k_offsets, B + 1, dev)
    a = _act(act)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    gdt = dtype if grad_dtype is None else grad_dtype
    if gdt not in DTYPE:
        raise ValueError(f"grad_dtype must be float32 or bfloat16, got {gdt}")
    if dq is None:
        dq = torch.empty((Tq, H, d), dtype=gdt, device=dev)
    else:
        _check("dq", dq, gdt, shape=(Tq, H, d), device=dev)
    if dk is None:
        dk = torch.empty((Tk, H, d), dtype=gdt, device=dev)
    else:
        _check("dk", dk, gdt, shape=(Tk, H, d), device=dev)
    if dv is None:
        dv = torch.empty((Tk, H, d), dtype=gdt, device=dev)
    else:
        _check("dv", dv, gdt, shape=(Tk, H, d), device=dev)
    ws_bytes = int(lib.ja_bwd_workspace_size(B, H, d, Tq, Tk, a, int(bool(causal)), int(window), DTYPE[dtype]))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, ws_bytes, dev)
    _disjoint(dict(dq=dq, dk=dk, dv=dv, workspace=workspace),
              dict(q=q, k=k, v=v, out=out, dout=dout, lse=lse, q_offsets=q_offsets, k_offsets=k_offsets))
    _on_gpu("q", q)
    status = lib.jagged_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(q_offsets),
                                 _ptr(k_offsets), B, H, d, Tq, Tk, a, int(bool(causal)), int(window),
                                 float(scale), DTYPE[dtype], DTYPE[gdt], _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(workspace), workspace.numel(), _stream(q.device, stream))
    _lib.check("jagged_attn_bwd", status)
    return dq, dk, dv


def block_attn_workspace_size(B, H, d, T, block, causal=False, dtype=torch.bfloat16) -> int:
    return int(_lib.load().ja_block_attn_workspace_size(B, H, d, T, int(block), int(bool(causal)), DTYPE[dtype]))


@_on_stream
def jagged_block_attn_fwd(q, k, v, offsets, block, causal=False, scale=None, out=None, lse=None,
                          workspace=None, stream=None, return_lse=True):
    """Block-diagonal self-attention forward (softmax): each block of ``block`` tokens
    of a sequence attends only within itself. q, k, v: [T,H,d]; offsets: int32 [B+1].

    Returns (out [T,H,d], lse [T,H] float32, or None with return_lse=False and no
    ``lse`` given)."""
    lib = _lib.load()
    if not isinstance(q, torch.Tensor) or q.dtype not in DTYPE:
        raise ValueError(f"q must be a float32 or bfloat16 tensor")
    _check("q", q, dim=3)
    dtype, dev = q.dtype, q.device
    T, H, d = q.shape
    _check("k", k, dtype, shape=(T, H, d), device=dev)
    _check("v", v, dtype, shape=(T, H, d), device=dev)
    if not isinstance(offsets, torch.Tensor) or offsets.dim() != 1 or offsets.numel() < 1:
        raise ValueError("offsets must be an int32 [B+1] tensor")
    B = offsets.numel() - 1
    _check_offsets("offsets", offsets, B + 1, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, dtype, shape=(T, H, d), device=dev)
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    elif lse is not None:
        _check("lse", lse, torch.float32, shape=(T, H), device=dev)
    ws_bytes = block_attn_workspace_size(B, H, d, T, block, causal, dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, ws_bytes, dev)
    _disjoint(dict(out=out, lse=lse, workspace=workspace), dict(q=q, k=k, v=v, offsets=offsets))
    _on_gpu("q", q)
    status = lib.jagged_block_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets), B, H, d, T, int(block),
                                       int(bool(causal)), float(scale), DTYPE[dtype], _ptr(out), _ptr(lse),
                                       _ptr(workspace), workspace.numel(), _stream(q.device, stream))
    _lib.check("jagged_block_attn_fwd", status)
    return out, lse


@_on_stream
def jagged_block_attn_bwd(q, k, v, out, dout, lse, offsets, block, causal=False, scale=None, dq=None, dk=None,
                          dv=None, workspace=None, stream=None):
    """Backward of jagged_block_attn_fwd. Returns (dq, dk, dv).

    For bf16 blocks of at most 64 tokens ``out`` and ``lse`` are not read (None is
    fine); larger blocks need the forward's."""
    lib = _lib.load()
    if not isinstance(q, torch.Tensor) or q.dtype not in DTYPE:
        raise ValueError(f"q must be a float32 or bfloat16 tensor")
    _check("q", q, dim=3)
    dtype, dev = q.dtype, q.device
    T, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        _check(name, t, dtype, shape=(T, H, d), device=dev)
    if out is not None:
        _check("out", out, dtype, shape=(T, H, d), device=dev)
    if lse is not None:
        _check("lse", lse, torch.float32, shape=(T, H), device=dev)
    if not isinstance(offsets, torch.Tensor) or offsets.dim() != 1 or offsets.numel() < 1:
        raise ValueError("offsets must be an int32 [B+1] tensor")
    B = offsets.numel() - 1
    _check_offsets("offsets", offsets, B + 1, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _check(name, t, dtype, shape=(T, H, d), device=dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = block_attn_workspace_size(B, H, d, T, block, causal, dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, ws_bytes, dev)
    _disjoint(dict(dq=dq, dk=dk, dv=dv, workspace=workspace),
              dict(q=q, k=k, v=v, out=out, dout=dout, lse=lse, offsets=offsets))
    _on_gpu("q", q)
    status = lib.jagged_block_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                       _ptr(offsets), B, H, d, T, int(block), int(bool(causal)), float(scale),
                                       DTYPE[dtype], _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                       workspace.numel(), _stream(q.device, stream))
    _lib.check("jagged_block_attn_bwd", status)
    return dq, dk, dv


@_on_stream
def mxfp8_quantize(x, offsets, stream=None):
    """MXFP8 quantization with [32, 32] blocks (32 tokens of one sequence x 32 channels
    of one head). x: bf16 [T,H,d] (d a multiple of 32); offsets: int32 [B+1].

    Returns (x8 uint8 [T,H,d] E4M3 codes, scales uint8 [NB,H,d/32] E8M0 exponents,
    scale_offsets int32 [B+1]); NB = ceil(T/32) + B rows are allocated, the first
    scale_offsets[B] are used."""
    lib = _lib.load()
    _check("x", x, torch.bfloat16, dim=3)
    T, H, d = x.shape
    if d % 32 != 0 or d < 32:
        raise ValueError(f"d must be a positive multiple of 32, got {d}")
    if not isinstance(offsets, torch.Tensor) or offsets.dim() != 1 or offsets.numel() < 1:
        raise ValueError("offsets must be an int32 [B+1] tensor")
    B = offsets.numel() - 1
    _check_offsets("offsets", offsets, B + 1, x.device)
    _on_gpu("x", x)
    nb = (T + 31) // 32 + B
    x8 = torch.empty((T, H, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((max(nb, 1), H, max(d // 32, 1)), dtype=torch.uint8, device=x.device)
    soff = torch.empty(B + 1, dtype=torch.int32, device=x.device)
    ws = torch.empty(max(int(lib.ja_mxfp8_quantize_workspace_size(B, T)), 256), dtype=torch.uint8, device=x.device)
    status = lib.ja_mxfp8_quantize(_ptr(x), DTYPE[torch.bfloat16], _ptr(offsets), B, H, d, T, _ptr(x8), _ptr(scales),
                                   _ptr(soff), _ptr(ws), ws.numel(), _stream(x.device, stream))
    _lib.check("ja_mxfp8_quantize", status)
    return x8, scales, soff


@_on_stream
def jagged_attn_fwd_mxfp8(q8, q_scales, q_scale_offsets, k8, k_scales, k_scale_offsets, v8, v_scales, q_offsets,
                          k_offsets, causal=False, window=0, scale=None, out=None, lse=None, workspace=None,
                          stream=None, return_lse=True):
    """Softmax attention forward on MXFP8 Q, K, V (from ``mxfp8_quantize``; K and V share
    k_scale_offsets), d = 128. Returns (out bf16 [Tq,H,d], lse [Tq,H] float32 or None)."""
    lib = _lib.load()
    _check("q8", q8, torch.uint8, dim=3)
    dev = q8.device
    Tq, H, d = q8.shape
    if not isinstance(k8, torch.Tensor) or k8.dim() != 3:
        raise ValueError("k8 must be a [Tk, H, d] tensor")
    Tk = k8.shape[0]
    _check("k8", k8, torch.uint8, shape=(Tk, H, d), device=dev)
    _check("v8", v8, torch.uint8, shape=(Tk, H, d), device=dev)
    if not isinstance(q_offsets, torch.Tensor) or q_offsets.dim() != 1 or q_offsets.numel() < 1:
        raise ValueError("q_offsets must be an int32 [B+1] tensor")
    B = q_offsets.numel() - 1
    for name, t in (("q_offsets", q_offsets), ("k_offsets", k_offsets), ("q_scale_offsets", q_scale_offsets),
                    ("k_scale_offsets", k_scale_offsets)):
        _check_offsets(name, t, B + 1, dev)
    # Scale rows: sequence b's blocks start at its scale offset; for offsets that are
    # consistent with the tensors that is at most ceil(T/32) + B rows in all (the
    # size mxfp8_quantize allocates), which every scale array must have.
    nbq, nbk = (Tq + 31) // 32 + B, (Tk + 31) // 32 + B
    for name, t, nb in (("q_scales", q_scales, nbq), ("k_scales", k_scales, nbk), ("v_scales", v_scales, nbk)):
        _check(name, t, torch.uint8, dim=3, device=dev)
        if t.shape[1:] != (H, d // 32) or t.shape[0] < max(nb, 1):
            raise ValueError(f"{name} must be [>= {max(nb, 1)}, {H}, {d // 32}], got {tuple(t.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((Tq, H, d), dtype=torch.bfloat16, device=dev)
    else:
        _check("out", out, torch.bfloat16, shape=(Tq, H, d), device=dev)
    if lse is None and return_lse:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
    elif lse is not None:
        _check("lse", lse, torch.float32, shape=(Tq, H), device=dev)
    ws_bytes = int(lib.ja_fwd_mxfp8_workspace_size(B, H, d, Tq, Tk))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    else:
        _check_workspace(workspace, ws_bytes, dev)
    _disjoint(dict(out=out, lse=lse, workspace=workspace),
              dict(q8=q8, q_scales=q_scales, k8=k8, k_scales=k_scales, v8=v8, v_scales=v_scales, q_offsets=q_offsets,
                   k_offsets=k_offsets, q_scale_offsets=q_scale_offsets, k_scale_offsets=k_scale_offsets))
    _on_gpu("q8", q8)
    status = lib.jagged_attn_fwd_mxfp8(_ptr(q8), _ptr(q_scales), _ptr(q_scale_offsets), _ptr(k8), _ptr(k_scales),
                                       _ptr(k_scale_offsets), _ptr(v8), _ptr(v_scales), _ptr(q_offsets),
                                       _ptr(k_offsets), B, H, d, Tq, Tk, int(bool(causal)), int(window), float(scale),
                                       _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                       _stream(q8.device, stream))
    _lib.check("jagged_attn_fwd_mxfp8", status)
    return out, lse


def fwd_tile_shape(B, d, Tq, Tk, act="softmax", dtype=torch.bfloat16):
    """(query rows per work item, keys per stage) of the forward for these sizes; the
    layout (standard, split for short queries, chunked for short keys) follows from B,
    Tq and Tk alone."""
    import ctypes
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    status = _lib.load().ja_fwd_tile_shape(B, d, Tq, Tk, _act(act), DTYPE[dtype], ctypes.byref(bm),
                                           ctypes.byref(bn))
    _lib.check("ja_fwd_tile_shape", status)
    return bm.value, bn.value


@_on_stream
def fwd_schedule(q_offsets, k_offsets, H, d, Tq, Tk, act="softmax", causal=False, window=0,
                 dtype=torch.bfloat16, stream=None):
    """Run only the forward's tile scheduler; returns the (sequence, tile) pairs as an int32 [n,2] GPU tensor."""
    lib = _lib.load()
    if not isinstance(q_offsets, torch.Tensor) or q_offsets.dim() != 1 or q_offsets.numel() < 1:
        raise ValueError("q_offsets must be an int32 [B+1] tensor")
    B = q_offsets.numel() - 1
    _check_offsets("q_offsets", q_offsets, B + 1, q_offsets.device)
    _check_offsets("k_offsets", k_offsets, B + 1, q_offsets.device)
    _on_gpu("q_offsets", q_offsets)
    bm, _ = fwd_tile_shape(B, d, Tq, Tk, act, dtype)
    max_items = (Tq + bm - 1) // bm + B
    items = torch.empty((max(max_items, 1), 2), dtype=torch.int32, device=q_offsets.device)
    count = torch.zeros(1, dtype=torch.int32, device=q_offsets.device)
    a = _act(act)
    ws_bytes = int(lib.ja_fwd_workspace_size(B, H, d, Tq, Tk, a, int(bool(causal)), int(window), DTYPE[dtype]))
    workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q_offsets.device)
    status = lib.ja_fwd_schedule(_ptr(q_offsets), _ptr(k_offsets), B, H, d, Tq, Tk, a, int(bool(causal)),
                                 int(window), DTYPE[dtype], _ptr(items), _ptr(count), max_items, _ptr(workspace),
                                 workspace.numel(), _stream(q_offsets.device, stream))
    _lib.check("ja_fwd_schedule", status)
    n = int(count.item())
    return items[:n]


@_on_stream
def validate_offsets(offsets, T, stream=None) -> bool:
    if not isinstance(offsets, torch.Tensor) or offsets.dim() != 1 or offsets.numel() < 1:
        raise ValueError("offsets must be an int32 [B+1] tensor")
    _check_offsets("offsets", offsets, offsets.numel(), offsets.device)
    _on_gpu("offsets", offsets)
    status = _lib.load().ja_validate_offsets(_ptr(offsets), offsets.numel() - 1, int(T),
                                             _stream(offsets.device, stream))
    if status == 4:
        return False
    _lib.check("ja_validate_offsets", status)
    return True
