"""ctypes loader for libjagged_attn.so (the C ABI in include/jagged_attn.h).

The library is built in-tree by ``jagged_attention_recsys_amd.build``. There is no
fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

# The in-tree build; JAGGED_ATTN_LIB may name another build of the same library.
LIB_PATH = os.environ.get("JAGGED_ATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "libjagged_attn.so")

# Symbols declared in include/jagged_attn.h, with their ctypes signatures.
_i32, _i64, _f32, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "ja_fwd_workspace_size": (_sz, [_i32, _i32, _i32, _i64, _i64, _i32, _i32, _i32, _i32]),
    "jagged_attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64, _i32, _i32, _i32, _f32,
                               _i32, _vp, _vp, _vp, _sz, _vp]),
    "jagged_attn_fwd_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64, _i32, _i32, _i32,
                                       _f32, _i32, _vp, _vp, _vp]),
    "ja_bwd_workspace_size": (_sz, [_i32, _i32, _i32, _i64, _i64, _i32, _i32, _i32, _i32]),
    "jagged_attn_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64, _i32, _i32,
                               _i32, _f32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ja_block_attn_workspace_size": (_sz, [_i32, _i32, _i32, _i64, _i32, _i32, _i32]),
    "jagged_block_attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i32, _i32, _f32, _i32, _vp, _vp,
                                     _vp, _sz, _vp]),
    "jagged_block_attn_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i32, _i32, _f32,
                                     _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ja_mxfp8_quantize_workspace_size": (_sz, [_i32, _i64]),
    "ja_mxfp8_quantize": (_i32, [_vp, _i32, _vp, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ja_fwd_mxfp8_workspace_size": (_sz, [_i32, _i32, _i32, _i64, _i64]),
    "jagged_attn_fwd_mxfp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64,
                                     _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "ja_fwd_schedule": (_i32, [_vp, _vp, _i32, _i32, _i32, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _i64,
                               _vp, _sz, _vp]),
    "ja_fwd_tile_shape": (_i32, [_i32, _i32, _i64, _i64, _i32, _i32, _vp, _vp]),
    "ja_validate_offsets": (_i32, [_vp, _i32, _i64, _vp]),
    "ja_set_profile_events": (None, [_vp, _vp]),
    "ja_set_profile_events3": (None, [_vp, _vp, _vp]),
    "ja_probe_mfma_workspace_size": (_sz, []),
    "ja_probe_mfma": (_i32, [_i32, _vp, _sz, _vp, _vp, _vp, _vp]),
    "ja_status_string": (ctypes.c_char_p, [_i32]),
    "ja_version": (_i32, []),
}

_lib = None


class JaggedAttnError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {status_string(status)} (status {status})")


def open_library(path: str) -> ctypes.CDLL:
    """Load a build of the library at `path` with the C signatures set."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m jagged_attention_recsys_amd.build` "
            "(hipcc, gfx950). There is no non-HIP fallback.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = open_library(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using(lib: ctypes.CDLL):
    """Route the binding's calls to another build of the library (tests compare builds)."""
    global _lib
    load()
    saved, _lib = _lib, lib
    try:
        yield lib
    finally:
        _lib = saved


def status_string(status: int) -> str:
    return load().ja_status_string(int(status)).decode()


def check(func: str, status: int) -> None:
    if status != 0:
        raise JaggedAttnError(func, status)
