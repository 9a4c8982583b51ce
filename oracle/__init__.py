"""fp64 CPU oracle for jagged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never imports, links or calls it, and the oracle imports
nothing from the product path.

The arithmetic lives in ``ja_oracle.c`` (plain C, fp64, libm only); this module
only builds it with gcc and marshals numpy arrays through ctypes. What it
computes is defined on the pages of the engineering post "GEM Training: How
Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model", sections
"Jagged Sequence Flash Attention", "Generalized Dot-Product Attention (GDPA)"
and "BlockAttention" (sliding window); the readings taken where the pages are
silent are listed in ``ja_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ja_oracle.c")
_LIB = os.path.join(_HERE, "libja_oracle.so")

SOFTMAX, SILU, GELU_TANH, GELU_TAYLOR = 0, 1, 2, 3
_DT_F32, _DT_BF16, _DT_F64 = 0, 1, 2
ACTS = {"softmax": SOFTMAX, "silu": SILU, "gelu": GELU_TANH, "gelu_tanh": GELU_TANH, "gelu_taylor": GELU_TAYLOR}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict IEEE order: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=gnu99", "-fPIC", "-shared", "-pthread",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        vp, i32p, u8p, f64p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        i32, f64, i64 = ctypes.c_int32, ctypes.c_double, ctypes.c_int64
        lib.ora_fwd_block.argtypes = [vp, vp, vp, ctypes.c_int, i32p, i32p, i32, i32, i32,
                                      ctypes.c_int, ctypes.c_int, i32, i32, f64, u8p, f64p, f64p, ctypes.c_int]
        lib.ora_fwd_block.restype = ctypes.c_int
        lib.ora_bwd_block.argtypes = [vp, vp, vp, vp, ctypes.c_int, i32p, i32p, i32, i32, i32,
                                      ctypes.c_int, ctypes.c_int, i32, i32, f64, u8p, f64p, f64p,
                                      f64p, f64p, f64p, ctypes.c_int]
        lib.ora_bwd_block.restype = ctypes.c_int
        lib.ora_tile_list_block.argtypes = [i32p, i32p, i32, i32, i32, ctypes.c_int, i32, i32,
                                            ctypes.c_int, i32, i32p, i32p, i64]
        lib.ora_tile_list_block.restype = ctypes.c_int64
        lib.ora_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.ora_e4m3_decode.restype = f64
        lib.ora_e4m3_encode.argtypes = [f64]
        lib.ora_e4m3_encode.restype = ctypes.c_uint8
        lib.ora_mxfp8_quantize.argtypes = [vp, ctypes.c_int, i32p, i32, i32, i32, u8p, u8p, i32p]
        lib.ora_mxfp8_quantize.restype = ctypes.c_int
        lib.ora_fwd_mxfp8.argtypes = [u8p, u8p, i32p, u8p, u8p, i32p, u8p, u8p, i32p, i32p, i32, i32, i32,
                                      ctypes.c_int, i32, f64, ctypes.c_int, u8p, f64p, f64p, ctypes.c_int]
        lib.ora_fwd_mxfp8.restype = ctypes.c_int
        lib.ora_num_threads.argtypes = []
        lib.ora_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().ora_num_threads())


def _as_input(x: np.ndarray):
    """Map a numpy array to (contiguous array, oracle dtype code). bf16 arrives as uint16 bits."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, _DT_F32
    if x.dtype == np.float64:
        return x, _DT_F64
    if x.dtype == np.uint16:
        return x, _DT_BF16
    raise TypeError(f"oracle input dtype {x.dtype} not supported (float32, float64, uint16=bf16 bits)")


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _offsets(off) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(off, dtype=np.int32))


def fwd(q, k, v, q_offsets, k_offsets, act="softmax", causal=False, window=0, scale=None,
        pair_mask=None, nthreads=0, block=0):
    """Forward oracle. q: [Tq,H,d]; k, v: [Tk,H,d] (float32, float64 or bf16 bits as uint16).

    ``block`` > 0 adds the block-diagonal mask (query i sees key j only if both lie
    in the same ``block``-token block of their sequence). Returns (out [Tq,H,d]
    float64, lse [Tq,H] float64). Rows of pairs not selected by ``pair_mask``
    ([B,H] bool) are NaN.
    """
    lib = _load()
    q, dt = _as_input(q)
    k, dtk = _as_input(k)
    v, dtv = _as_input(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share a dtype")
    qo, ko = _offsets(q_offsets), _offsets(k_offsets)
    B = qo.shape[0] - 1
    Tq, H, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.full((Tq, H, d), np.nan, dtype=np.float64)
    lse = np.full((Tq, H), np.nan, dtype=np.float64)
    pm = None if pair_mask is None else np.ascontiguousarray(np.asarray(pair_mask, dtype=np.uint8).reshape(-1))
    rc = lib.ora_fwd_block(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(qo), _ptr(ko), B, H, d,
                           ACTS[act] if isinstance(act, str) else int(act), int(bool(causal)), int(window),
                           int(block), float(scale), _ptr(pm), _ptr(out), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, lse


def bwd(q, k, v, dout, q_offsets, k_offsets, act="softmax", causal=False, window=0, scale=None,
        pair_mask=None, nthreads=0, block=0):
    """Backward oracle. Returns (out, lse, dq, dk, dv) as float64 arrays (NaN outside pair_mask)."""
    lib = _load()
    q, dt = _as_input(q)
    k, _ = _as_input(k)
    v, _ = _as_input(v)
    dout, dt2 = _as_input(dout)
    if dt2 != dt:
        raise TypeError("dout must share the dtype of q")
    qo, ko = _offsets(q_offsets), _offsets(k_offsets)
    B = qo.shape[0] - 1
    Tq, H, d = q.shape
    Tk = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.full((Tq, H, d), np.nan)
    lse = np.full((Tq, H), np.nan)
    dq = np.full((Tq, H, d), np.nan)
    dk = np.full((Tk, H, d), np.nan)
    dv = np.full((Tk, H, d), np.nan)
    pm = None if pair_mask is None else np.ascontiguousarray(np.asarray(pair_mask, dtype=np.uint8).reshape(-1))
    rc = lib.ora_bwd_block(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), dt, _ptr(qo), _ptr(ko), B, H, d,
                           ACTS[act] if isinstance(act, str) else int(act), int(bool(causal)), int(window),
                           int(block), float(scale), _ptr(pm), _ptr(out), _ptr(lse), _ptr(dq), _ptr(dk),
                           _ptr(dv), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, lse, dq, dk, dv


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 codes (ties to even) of values in [-448, 448]."""
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    return np.array([lib.ora_e4m3_encode(float(v)) for v in x.reshape(-1)], dtype=np.uint8).reshape(x.shape)


def e4m3_decode(b) -> np.ndarray:
    lib = _load()
    b = np.asarray(b, dtype=np.uint8)
    return np.array([lib.ora_e4m3_decode(int(v)) for v in b.reshape(-1)], dtype=np.float64).reshape(b.shape)


def mxfp8_quantize(x, offsets, block_rows: int = 32):
    """MXFP8 with [32, 32] blocks per sequence and head: returns (x8 [T,H,d] uint8 E4M3
    codes, scales [NB,H,d/32] uint8 E8M0, soff [B+1] int32 first block of each sequence)."""
    assert block_rows == 32
    lib = _load()
    x, dt = _as_input(x)
    off = _offsets(offsets)
    B = off.shape[0] - 1
    T, H, d = x.shape
    soff = np.zeros(B + 1, dtype=np.int32)
    nb = int(np.sum((np.diff(off.astype(np.int64)) + 31) // 32))
    x8 = np.zeros((T, H, d), dtype=np.uint8)
    scales = np.zeros((max(nb, 1), H, d // 32), dtype=np.uint8)
    rc = lib.ora_mxfp8_quantize(_ptr(x), dt, _ptr(off), B, H, d, _ptr(x8), _ptr(scales), _ptr(soff))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return x8, scales[:nb], soff


def fwd_mxfp8(q8, qs, q_soff, k8, ks, k_soff, v8, vs, q_offsets, k_offsets, causal=False, window=0,
              scale=None, pquant=True, pair_mask=None, nthreads=0):
    """Softmax attention forward on MXFP8 inputs (K and V share k_soff); with pquant the
    softmax weights are rounded to E4M3 at scale 2^-8 before P V. Returns (out, lse) float64."""
    lib = _load()
    arrs = [np.ascontiguousarray(a, dtype=np.uint8) for a in (q8, qs, k8, ks, v8, vs)]
    q8, qs, k8, ks, v8, vs = arrs
    qso, kso = _offsets(q_soff), _offsets(k_soff)
    qo, ko = _offsets(q_offsets), _offsets(k_offsets)
    B = qo.shape[0] - 1
    Tq, H, d = q8.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.full((Tq, H, d), np.nan, dtype=np.float64)
    lse = np.full((Tq, H), np.nan, dtype=np.float64)
    pm = None if pair_mask is None else np.ascontiguousarray(np.asarray(pair_mask, dtype=np.uint8).reshape(-1))
    rc = lib.ora_fwd_mxfp8(_ptr(q8), _ptr(qs), _ptr(qso), _ptr(k8), _ptr(ks), _ptr(kso), _ptr(v8), _ptr(vs),
                           _ptr(qo), _ptr(ko), B, H, d, int(bool(causal)), int(window), float(scale),
                           int(bool(pquant)), _ptr(pm), _ptr(out), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, lse


def tile_list(row_offsets, col_offsets, BM, BN, causal=False, window=0, transposed=False, cap=1 << 30,
              block=0):
    """Reference work list: (items [n,2] int32 of (b, tile), costs [n] int32), sorted by
    min(cost, cap) descending, then b, then tile ascending."""
    lib = _load()
    ro, co = _offsets(row_offsets), _offsets(col_offsets)
    B = ro.shape[0] - 1
    L = np.diff(ro.astype(np.int64))
    nmax = int(np.sum((L + BM - 1) // BM)) if B > 0 else 0
    items = np.zeros((max(nmax, 1), 2), dtype=np.int32)
    costs = np.zeros(max(nmax, 1), dtype=np.int32)
    n = lib.ora_tile_list_block(_ptr(ro), _ptr(co), B, int(BM), int(BN), int(bool(causal)), int(window),
                                int(block), int(bool(transposed)), int(cap), _ptr(items), _ptr(costs), nmax)
    if n < 0:
        raise ValueError("oracle rejected the arguments")
    return items[:n].copy(), costs[:n].copy()
