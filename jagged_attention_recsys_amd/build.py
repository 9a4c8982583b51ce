"""Build libjagged_attn.so (HIP, gfx950) in-tree.

Every translation unit under ``csrc/`` is compiled with hipcc for gfx950 only, in
parallel, then linked into ``libjagged_attn.so`` next to this file. Packed-FP32
instruction selection is switched off for the device code.

    python -m jagged_attention_recsys_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libjagged_attn.so")
# Race-check build: every stage streamed through one LDS buffer (JA_SINGLE_STAGE);
# tests require its results to equal the normal build's bit for bit.
LIB_SINGLE_STAGE = os.path.join(PKG, "libjagged_attn_single_stage.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def common_flags() -> list[str]:
    # The atomic optimizer would wrap the forward's single-lane work-queue pop in
    # wave-wide bookkeeping that waits for the atomic's return on the spot; the pop
    # is issued before an item's epilogue and its result is read after it.
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-I", INCLUDE, "-I", CSRC]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, build_dir: str = BUILD_DIR, defines: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *common_flags(), *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _build_one(lib: str, build_dir: str, defines: tuple, jobs: int | None, verbose: bool) -> str:
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), srcs))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(verbose: bool = False, jobs: int | None = None, single_stage: bool = True) -> str:
    """Compile every source and link the shared library (and, unless single_stage is
    False, the single-stage race-check build beside it); returns the library's path."""
    _build_one(LIB, BUILD_DIR, (), jobs, verbose)
    if single_stage:
        _build_one(LIB_SINGLE_STAGE, os.path.join(BUILD_DIR, "single_stage"), ("JA_SINGLE_STAGE=1",), jobs, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
