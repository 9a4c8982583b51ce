"""The machine probe behind the bench line's sustained matrix rate and clock
(ja_probe_mfma): one workgroup per compute unit, the stated matrix work per
workgroup, per-workgroup cycle and tick counts that give a plausible shader clock,
a rate below the chip's dense bf16 peak, and its argument errors."""
import ctypes

import numpy as np
import pytest
import torch

from jagged_attention_recsys_amd import _lib

pytestmark = pytest.mark.gpu

PEAK_BF16_TFLOPS = 2500.0
JA_ERR_INVALID_ARG, JA_ERR_WORKSPACE = 1, 3


def _probe(lib, iters, ws, nbytes):
    groups, fpg, khz = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
    st = lib.ja_probe_mfma(iters, ws.data_ptr() if ws is not None else None, nbytes, ctypes.byref(groups),
                           ctypes.byref(fpg), ctypes.byref(khz), torch.cuda.current_stream().cuda_stream)
    return st, groups.value, fpg.value, khz.value


def test_probe_counts_and_rate():
    lib = _lib.load()
    nbytes = int(lib.ja_probe_mfma_workspace_size())
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    iters = 4000
    assert _probe(lib, iters // 4, ws, nbytes)[0] == 0  # warm the clock
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    st, groups, fpg, khz = _probe(lib, iters, ws, nbytes)
    e1.record()
    torch.cuda.synchronize()
    assert st == 0
    assert groups == torch.cuda.get_device_properties(0).multi_processor_count
    # four waves, four independent 32x32x16 products each per round, 2*32*32*16 flop per product
    assert fpg == iters * 4 * 4 * 2 * 32 * 32 * 16
    assert khz > 0
    t = ws[: 16 * groups].cpu().view(torch.int64).numpy().reshape(-1, 2).astype(np.float64)
    assert np.all(t[:, 0] > 0) and np.all(t[:, 1] > 0)
    mhz = t[:, 0] / (t[:, 1] / (khz * 1e3)) / 1e6
    assert np.all((mhz > 300) & (mhz < 3000)), f"implausible shader clocks {mhz.min():.0f}..{mhz.max():.0f} MHz"
    tflops = groups * fpg / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert 0 < tflops <= PEAK_BF16_TFLOPS * 1.02, f"{tflops:.0f} TFLOP/s"


def test_probe_argument_errors():
    lib = _lib.load()
    nbytes = int(lib.ja_probe_mfma_workspace_size())
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    assert _probe(lib, 0, ws, nbytes)[0] == JA_ERR_INVALID_ARG
    assert _probe(lib, 10, None, nbytes)[0] == JA_ERR_INVALID_ARG
    assert _probe(lib, 10, ws, nbytes - 1)[0] == JA_ERR_WORKSPACE
    torch.cuda.synchronize()
