#!/usr/bin/env python3
"""Throughput of the jagged attention hot path on one MI355X; prints ONE JSON line.

A step is one pass of the whole hot path over one resident synthetic batch: by
default the long sliding-window causal softmax self-attention batch (B=32, lengths
lognormal with median 2048 capped at 32768, window 1024, H=8, d=128, bf16), forward
AND backward, i.e. ``jagged_attn_fwd`` (device tile scheduler + fused forward) then
``jagged_attn_bwd`` (two schedulers, the dQ pass with its Di prologue, the dK/dV
pass). ``--workload 2|3|4|6|7|8`` measures the other batches (forward only unless
``--bwd``; 6 and 7 include their backward like 5; ``--fwd-only`` drops it);
``--act`` swaps the activation.

Before the warm-up steps the step runs untimed for --spinup-ms (default 200 ms): an
idle GPU takes tens of milliseconds of load to reach its working clock.

Reported:
  value        useful (unpadded) TFLOP/s of the whole step: 4 d H sum_b pairs_b for
               the forward plus 10 d H pairs for the backward (the FlashAttention
               convention), pairs_b = visible (query, key) pairs of sequence b, over
               the wall-clock step time (K steps between two synchronisations);
  step_ms      median / min / max of the per-step HIP-event durations;
  fwd, bwd     each phase's kernels alone (HIP events the library records on its
               stream right around them): forward TFLOP/s (the metric's own phase)
               and its fraction of the dense bf16 peak; the dQ and dK/dV passes;
  roofline     the dominant kernel of the step (longest median duration): its
               algorithmic flop (forward 4 d, dQ pass 6 d, dK/dV pass 8 d per
               visible pair and head: the products each kernel must form from its
               inputs) or algorithmic bytes (inputs read and outputs written once)
               per launch over its median duration, against the published peak its
               arithmetic intensity makes binding (dense bf16 2.5 PFLOP/s, HBM 8
               TB/s); `traffic` is HBM bytes per launch from committed rocprofv3
               counter runs, or null when the kernel source changed since;
  machine      the bf16 matrix rate a plain stream of products sustains on every
               SIMD and the shader clock meanwhile (library probe, same run);
  cpu_baseline the fp64 oracle on a bounded sample of the same batch, on every host
               core (a reported baseline, not a target); its outputs double as a
               parity spot-check of the GPU result on the sampled pairs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak (published)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop per byte where the two peaks meet
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "ja_fwd_kernel": ["ja_fwd.hip", "ja_common.h", "ja_lds.h", "ja_tiles.h", "ja_internal.h"],
    "ja_mx_fwd_kernel": ["ja_mx.hip", "ja_mx.h", "ja_common.h", "ja_lds.h", "ja_tiles.h", "ja_internal.h"],
    "ja_bwd_dq_kernel": ["ja_bwd.hip", "ja_common.h", "ja_lds.h", "ja_tiles.h", "ja_internal.h"],
    "ja_bwd_dkdv_kernel": ["ja_bwd.hip", "ja_common.h", "ja_lds.h", "ja_tiles.h", "ja_internal.h"],
    "ja_blk_bwd_kernel": ["ja_block.hip", "ja_block.h", "ja_common.h", "ja_lds.h", "ja_tiles.h", "ja_internal.h"],
}
METRIC = "useful (unpadded) bf16 TFLOP/s of jagged attn fwd; % of MI355X MFMA peak"
FWD_BWD_WORKLOADS = (5, 6, 7)  # batches whose configuration is forward + backward


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def visible_pairs(lq: np.ndarray, lk: np.ndarray, causal: bool, window: int, block: int = 0) -> int:
    """Exact number of visible (query, key) pairs of a jagged batch (block > 0: the
    block-diagonal self-attention mask, blocks of `block` tokens)."""
    total = 0
    for Lq, Lk in zip(lq.tolist(), lk.tolist()):
        if Lq <= 0 or Lk <= 0:
            continue
        if block > 0:  # self-attention: full blocks plus one short last block
            sizes = [block] * (Lq // block) + ([Lq % block] if Lq % block else [])
            total += sum(g * (g + 1) // 2 if causal else g * g for g in sizes)
            continue
        if not causal and window == 0:
            total += Lq * Lk
            continue
        i = np.arange(Lq, dtype=np.int64)
        lo = np.zeros(Lq, dtype=np.int64) if window == 0 else np.maximum(0, i - window + 1)
        if causal:
            hi = np.minimum(i, Lk - 1)
        else:
            hi = np.full(Lq, Lk - 1, dtype=np.int64) if window == 0 else np.minimum(Lk - 1, i + window - 1)
        total += int(np.maximum(0, hi - lo + 1).sum())
    return total


def kernel_work(name: str, w, pairs: int, Tq: int, Tk: int, need_lse: bool):
    """(algorithmic flop, algorithmic bytes) of one launch of kernel `name` on batch w:
    the matrix products the kernel must form from its inputs, and its inputs read
    and outputs written once."""
    e = 2 if w.dtype == "bf16" else 4
    row = w.H * w.d * e  # bytes of one token row of one tensor
    softmax = w.act == "softmax"
    if name in ("ja_fwd_kernel", "ja_mx_fwd_kernel"):
        if name == "ja_mx_fwd_kernel":
            row = w.H * w.d  # one byte per element (plus block scales, 1/32 of that, left out)
        flop = 4.0 * w.d * w.H * pairs
        byts = row * (Tq + 2 * Tk) + 2 * w.H * w.d * Tq + (4 * w.H * Tq if need_lse else 0)
    elif name == "ja_bwd_dq_kernel":
        flop = 6.0 * w.d * w.H * pairs                      # S, dP, dQ
        byts = row * (2 * Tq + 2 * Tk) + row * Tq           # Q, dO, K, V in; dQ out
        if softmax:
            byts += row * Tq + 4 * w.H * Tq + 4 * w.H * Tq  # O, lse in; Di out
    elif name == "ja_bwd_dkdv_kernel":
        flop = 8.0 * w.d * w.H * pairs                      # S, dP, dV, dK
        byts = row * (2 * Tk + 2 * Tq) + 2 * row * Tk       # K, V, Q, dO in; dK, dV out
        if softmax:
            byts += 8 * w.H * Tq                            # lse, Di in
    elif name == "ja_blk_bwd_kernel":
        flop = 10.0 * w.d * w.H * pairs                     # S, dP, dV, dK, dQ in one pass
        byts = row * 4 * Tq + row * 3 * Tq                  # Q, K, V, dO in; dQ, dK, dV out
    else:
        raise ValueError(name)
    return flop, float(byts)


def kernel_sha(name: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        p = os.path.join(ROOT, "jagged_attention_recsys_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()


def recorded_traffic(name: str, workload: str):
    """HBM bytes per launch from committed counter runs, if taken on the current kernel source."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = data.get(name, {}).get(workload)
    if not rec or rec.get("source_sha256") != kernel_sha(name):
        return None
    return rec.get("hbm_bytes_per_launch")


def _stats(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(xs)), 4), "min": round(float(xs.min()), 4),
            "max": round(float(xs.max()), 4)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5, choices=[2, 3, 4, 5, 6, 7, 8])
    ap.add_argument("--bwd", action="store_true", help="add the backward to a forward-only batch (2, 3, 4)")
    ap.add_argument("--fwd-only", action="store_true", help="drop the backward of batches 5, 6, 7")
    ap.add_argument("--act", choices=["softmax", "silu", "gelu", "gelu_taylor"], default=None,
                    help="run the workload with another activation (e.g. 7 with the tanh GELU)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle budget for the CPU baseline")
    ap.add_argument("--spinup-ms", type=float, default=200.0,
                    help="untimed load before the warm-up steps, so the GPU has left its idle clock state")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the machine probe (sustained MFMA rate, clock)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy (y = x * 1) of MIB MiB, 5 times: the reference "
                         "for scaling HBM byte counters")
    ap.add_argument("--record-traffic", nargs=5,
                    metavar=("KERNEL", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="no GPU: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of --workload (and of "
                         "--copy-calibration 1024) into HBM bytes per launch of KERNEL in profiles/traffic.json")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.record_traffic:
        return record_traffic(args.workload, *args.record_traffic)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library runs the attention path on a single MI355X and has "
              "no multi-GPU path (each sequence and head is independent, so a batch would be sharded by "
              "sequence). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import jagged_attention_recsys_amd as ja
    from jagged_attention_recsys_amd import _lib
    from jagged_attention_recsys_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    lib = _lib.load()  # raises if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    do_bwd = (args.workload in FWD_BWD_WORKLOADS or args.bwd) and not args.fwd_only
    log(f"[bench] generating workload {args.workload}")
    w = W.workload(args.workload, act=args.act)
    if do_bwd and w.dout is None:
        W.with_upstream_gradient(w, 1000 + args.workload)  # seeded dO for the batches that draw none

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        return t.to(dev)

    q, k, v = up(w.q), up(w.k), up(w.v)
    qo, ko = up(w.q_offsets), up(w.k_offsets)
    dout = up(w.dout) if do_bwd else None
    mx = bool(w.extra.get("mxfp8"))
    if mx:
        if do_bwd:
            print("the MXFP8 path has no backward", file=sys.stderr)
            return 2
        # Quantized once, outside the timed steps (upstream kernels emit MXFP8).
        qm = ja.mxfp8_quantize(q, qo)
        km = ja.mxfp8_quantize(k, ko)
        vm = ja.mxfp8_quantize(v, ko)
    Tq, Tk = q.shape[0], k.shape[0]
    out = torch.empty_like(q)
    # The block path (blocks of at most 64 tokens) keeps no log-sum-exp: its
    # backward recomputes each block's softmax.
    fused_block = bool(w.block and w.block <= 64)
    need_lse = w.act == "softmax" and not fused_block
    lse = torch.empty((Tq, w.H), dtype=torch.float32, device=dev) if need_lse else None
    if mx:
        ws_fwd, ws_bwd = int(lib.ja_fwd_mxfp8_workspace_size(w.B, w.H, w.d, Tq, Tk)), 0
    elif w.block:
        ws_fwd = ws_bwd = ja.block_attn_workspace_size(w.B, w.H, w.d, Tq, w.block, w.causal)
    else:
        ws_fwd = ja.fwd_workspace_size(w.B, w.H, w.d, Tq, Tk, w.act, w.causal, w.window)
        ws_bwd = ja.bwd_workspace_size(w.B, w.H, w.d, Tq, Tk, w.act, w.causal, w.window) if do_bwd else 0
    ws = torch.empty(max(ws_fwd, 256), dtype=torch.uint8, device=dev)
    if do_bwd:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(max(ws_bwd, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    pairs = visible_pairs(w.lq, w.lk, w.causal, w.window, w.block)
    fwd_flop = 4.0 * w.d * w.H * pairs
    bwd_flop = 10.0 * w.d * w.H * pairs if do_bwd else 0.0
    fwd_name = "ja_mx_fwd_kernel" if mx else "ja_fwd_kernel"
    bwd_names = (["ja_blk_bwd_kernel"] if fused_block else ["ja_bwd_dq_kernel", "ja_bwd_dkdv_kernel"]) if do_bwd \
        else []

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
            lib.ja_set_profile_events(ev[1].cuda_event, ev[2].cuda_event)
        if mx:
            ja.jagged_attn_fwd_mxfp8(qm[0], qm[1], qm[2], km[0], km[1], km[2], vm[0], vm[1], qo, ko,
                                     causal=w.causal, window=w.window, scale=w.scale, out=out, lse=lse,
                                     workspace=ws, stream=stream)
        elif w.block:
            ja.jagged_block_attn_fwd(q, k, v, qo, w.block, causal=w.causal, scale=w.scale, out=out, lse=lse,
                                     workspace=ws, stream=stream, return_lse=need_lse)
        else:
            ja.jagged_attn_fwd(q, k, v, qo, ko, act=w.act, causal=w.causal, window=w.window, scale=w.scale,
                               out=out, lse=lse, workspace=ws, stream=stream)
        if do_bwd:
            if ev is not None:
                lib.ja_set_profile_events3(ev[3].cuda_event, ev[4].cuda_event if not fused_block else None,
                                           ev[5].cuda_event)
            if w.block:
                ja.jagged_block_attn_bwd(q, k, v, out, dout, lse, qo, w.block, causal=w.causal, scale=w.scale,
                                         dq=dq, dk=dk, dv=dv, workspace=bws, stream=stream)
            else:
                ja.jagged_attn_bwd(q, k, v, out, dout, lse, qo, ko, act=w.act, causal=w.causal, window=w.window,
                                   scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=bws, stream=stream)
        if ev is not None:
            lib.ja_set_profile_events(None, None)
            ev[6].record(stream)

    log(f"[bench] spin-up {args.spinup_ms:.0f} ms, then warmup {args.warmup} steps")
    t_end = time.perf_counter() + args.spinup_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per step: [step start, fwd before, fwd after, bwd before, bwd mid, bwd after, step end]
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for evs in events:  # create the underlying HIP events before handing them to the library
        for e in evs:
            e.record(stream)
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    step_ms = [e[0].elapsed_time(e[6]) for e in events]
    kms = {fwd_name: [e[1].elapsed_time(e[2]) for e in events]}
    if do_bwd:
        if fused_block:
            kms["ja_blk_bwd_kernel"] = [e[3].elapsed_time(e[5]) for e in events]
        else:
            kms["ja_bwd_dq_kernel"] = [e[3].elapsed_time(e[4]) for e in events]
            kms["ja_bwd_dkdv_kernel"] = [e[4].elapsed_time(e[5]) for e in events]
    med = {n: float(np.median(x)) for n, x in kms.items()}
    total_flop = fwd_flop + bwd_flop
    value = total_flop / (ms_per_step * 1e-3) / 1e12
    peak_mm = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS

    def roofline_of(name):
        flop, byts = kernel_work(name, w, pairs, Tq, Tk, need_lse)
        t = med[name] * 1e-3
        intensity = flop / byts
        r = {"kernel": name, "kernel_ms": round(med[name], 4), "flop_per_launch": flop, "bytes_per_launch": byts,
             "intensity_flop_per_byte": round(intensity, 1)}
        if intensity >= RIDGE:
            a = flop / t / 1e12
            r.update({"bound": "mfma", "achieved": round(a, 2), "peak": peak_mm, "unit": "TFLOP/s",
                      "frac": round(a / peak_mm, 4)})
        else:
            a = byts / t / 1e9
            r.update({"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(a / PEAK_HBM_GBS, 4), "tflops": round(flop / t / 1e12, 2)})
        r["traffic"] = recorded_traffic(name, f"w{args.workload}" + ("+bwd" if name != fwd_name else ""))
        return r

    dominant = max(med, key=lambda n: med[n])
    roofline = roofline_of(dominant)
    fwd_t = med[fwd_name] * 1e-3
    fwd = {"kernel": fwd_name, "kernel_ms": _stats(kms[fwd_name]),
           "tflops": round(fwd_flop / fwd_t / 1e12, 2), "frac_of_peak": round(fwd_flop / fwd_t / 1e12 / peak_mm, 4),
           "roofline": roofline_of(fwd_name) if dominant != fwd_name else "as roofline"}
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spinup_ms": args.spinup_ms,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": _stats(step_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "pct_of_peak": round(100.0 * value / peak_mm, 2),
        "dtype": "fp8-e4m3 (MX, [32,32] block scales)" if mx else "bf16",
        "data": "synthetic",
        "config": {"workload": w.extra.get("description", w.name), "B": w.B, "H": w.H, "d": w.d,
                   "act": w.act, "causal": bool(w.causal), "window": int(w.window), "block": int(w.block),
                   "scale": round(w.scale, 6), "q_tokens": int(Tq), "kv_tokens": int(Tk),
                   "visible_pairs": int(pairs), "fwd_flop": fwd_flop, "bwd_flop": bwd_flop,
                   "phases": "fwd+bwd" if do_bwd else "fwd"},
        "roofline": roofline,
        "fwd": fwd,
    }
    if do_bwd:
        bt = sum(med[n] for n in bwd_names) * 1e-3
        bwd = {"kernels_ms": round(bt * 1e3, 4), "tflops": round(bwd_flop / bt / 1e12, 2),
               "frac_of_peak": round(bwd_flop / bt / 1e12 / PEAK_BF16_TFLOPS, 4), "flop_convention": "10 d H pairs"}
        for n in bwd_names:
            bwd[n] = {"kernel_ms": _stats(kms[n])}
            if n != dominant:
                bwd[n]["roofline"] = roofline_of(n)
        result["bwd"] = bwd
    if roofline["bound"] == "hbm":
        copy = measure_copy_gbs(1024)  # what a plain streaming kernel sustains on this GPU, same run
        roofline["copy_gbs"] = round(copy, 1)
        roofline["frac_of_copy"] = round(roofline["achieved"] / copy, 4)
    if not args.no_probe:
        result["machine"] = machine_probe(lib, torch, stream)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, out, lse, (dq, dk, dv) if do_bwd and not w.block else None,
                                              args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def machine_probe(lib, torch, stream, iters: int = 20000) -> dict:
    """Sustained dense bf16 matrix rate and shader clock (ja_probe_mfma), event-timed."""
    import ctypes

    nbytes = int(lib.ja_probe_mfma_workspace_size())
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    groups, fpg, khz = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()

    def run(n):
        st = lib.ja_probe_mfma(n, ws.data_ptr(), nbytes, ctypes.byref(groups), ctypes.byref(fpg), ctypes.byref(khz),
                               int(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"ja_probe_mfma failed: {st}")

    run(iters // 4)  # warm
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run(iters)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ticks = ws[: 16 * groups.value].cpu().view(torch.int64).numpy().reshape(-1, 2).astype(np.float64)
    mhz = np.median(ticks[:, 0] / (ticks[:, 1] / (khz.value * 1e3))) / 1e6
    tflops = groups.value * fpg.value / (ms * 1e-3) / 1e12
    return {"sustained_mfma_bf16_tflops": round(tflops, 1), "sustained_frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "sclk_mhz_under_mfma": round(float(mhz), 0), "probe_ms": round(ms, 3), "workgroups": groups.value,
            "method": "ja_probe_mfma: one 4-wave workgroup per CU, 4 independent 32x32x16 bf16 chains per wave, "
                      f"{iters} rounds; clock = shader cycles / real-time ticks of the loop (median over CUs)"}


def _counter_per_dispatch(run_dir: str, counter: str, kernel_part: str) -> list[float]:
    """Counter values (summed over the rows of each dispatch) of the dispatches whose
    kernel name contains kernel_part, from a rocprofv3 --output-format csv run."""
    import csv
    import glob

    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel_part in r["Kernel_Name"]:
                key = (f, r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def record_traffic(workload: int, kernel: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str,
                   copy_write_dir: str) -> int:
    """HBM bytes per launch of `kernel` = FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled so that the copy kernel of known size reads and writes exactly its bytes."""
    if kernel not in KERNEL_SOURCES:
        raise SystemExit(f"unknown kernel {kernel}")
    copy_bytes = 1024 * (1 << 20)
    cf = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "elementwise")
    cw = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "elementwise")
    kf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", kernel)
    kw = _counter_per_dispatch(write_dir, "WRITE_SIZE", kernel)
    if not (cf and cw and kf and kw):
        raise SystemExit("missing dispatches in the counter runs")
    f_scale = copy_bytes / (float(np.median(cf)) * 1024.0)
    w_scale = copy_bytes / (float(np.median(cw)) * 1024.0)
    fetch = float(np.median(kf)) * 1024.0 * f_scale
    write = float(np.median(kw)) * 1024.0 * w_scale
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        data = {}
    fwd = kernel in ("ja_fwd_kernel", "ja_mx_fwd_kernel")
    key = f"w{workload}" + ("" if fwd else "+bwd")
    data.setdefault(kernel, {})[key] = {
        "hbm_bytes_per_launch": round(fetch + write),
        "fetch_bytes": round(fetch), "write_bytes": round(write),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "source_sha256": kernel_sha(kernel),
        "method": "rocprofv3 --pmc FETCH_SIZE then --pmc WRITE_SIZE on bench.py --workload "
                  f"{workload} --steps 2 --warmup 1 --no-cpu-baseline --no-probe; KiB per dispatch (median) x 1024 x "
                  "scale, scale = 1 GiB / the same counter on bench.py --copy-calibration 1024",
    }
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(data[kernel][key]))
    return 0


def measure_copy_gbs(mib: int, x=None, y=None) -> float:
    """Bytes read + written per second by a plain streaming kernel (y = x * 1 over mib MiB),
    20 event-timed launches after a 200 ms spin-up."""
    import torch

    n = mib * (1 << 20) // 4
    if x is None:
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    e1.record()
    torch.cuda.synchronize()
    return 2 * n * 4 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9


def copy_calibration(mib: int) -> int:
    """A plain streaming kernel of known traffic: reads and writes mib MiB per launch.
    Five launches serve as the counter calibration; the copy bandwidth the GPU
    sustains is then timed on the same buffers."""
    import torch

    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    gbs = measure_copy_gbs(mib, x, y)
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": 5, "copy_gbs": round(gbs, 1)}), flush=True)
    return 0


def cpu_baseline(w, out_gpu, lse_gpu, grads_gpu, budget_s: float) -> dict:
    """Time the fp64 oracle on a bounded sample of (sequence, head) pairs of the batch:
    the same step as the GPU's (forward, or forward + backward when grads_gpu is given),
    counted in the same useful flop."""
    import oracle  # test infrastructure: used here for the CPU baseline only

    with_bwd = grads_gpu is not None
    if w.extra.get("mxfp8"):
        # the MXFP8 forward on the oracle's quantization of the batch (bit-identical to
        # the library's, which the tests check); the quantization itself is upstream
        qm = oracle.mxfp8_quantize(w.q, w.q_offsets)
        km = oracle.mxfp8_quantize(w.k, w.k_offsets)
        vm = oracle.mxfp8_quantize(w.v, w.k_offsets)

        def run_oracle(mask):
            return oracle.fwd_mxfp8(qm[0], qm[1], qm[2], km[0], km[1], km[2], vm[0], vm[1], w.q_offsets,
                                    w.k_offsets, w.causal, w.window, w.scale, pquant=True, pair_mask=mask)
    elif with_bwd:
        def run_oracle(mask):  # (out, lse, dq, dk, dv)
            return oracle.bwd(w.q, w.k, w.v, w.dout, w.q_offsets, w.k_offsets, w.act, w.causal, w.window, w.scale,
                              pair_mask=mask, block=w.block)
    else:
        def run_oracle(mask):
            return oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, w.act, w.causal, w.window, w.scale,
                              pair_mask=mask, block=w.block)

    per_pair = (4.0 + (10.0 if with_bwd else 0.0)) * w.d
    rng = np.random.default_rng(1234)
    B, H = w.B, w.H
    order = [(int(b), int(h)) for b in rng.permutation(B) for h in range(H)]
    pair_flop = np.array([per_pair * visible_pairs(w.lq[b:b + 1], w.lk[b:b + 1], w.causal, w.window, w.block)
                          for b, _ in order])
    # Calibrate the oracle's rate on a growing prefix of the pair order (at least
    # ~1 s of work), then fill the budget.
    # (at least one pair per oracle thread, so the calibration runs as parallel as the sample)
    mask = np.zeros((B, H), dtype=bool)
    rate, n_cal = None, max(1, oracle.num_threads())
    while rate is None:
        mask[:] = False
        for b, h in order[:n_cal]:
            mask[b, h] = True
        t = time.perf_counter()
        run_oracle(mask)
        dt = time.perf_counter() - t
        if dt >= 2.0 or n_cal >= len(order):
            rate = max(pair_flop[:n_cal].sum(), 1.0) / max(dt, 1e-4)
        n_cal *= 2
    budget_flop = rate * budget_s
    mask[:] = False
    acc = 0.0
    for i, (b, h) in enumerate(order):
        if acc > 0 and acc + pair_flop[i] > budget_flop:
            continue
        mask[b, h] = True
        acc += pair_flop[i]
    log(f"[bench] cpu baseline: {int(mask.sum())} pairs, {acc:.3g} flop")
    t = time.perf_counter()
    res = run_oracle(mask)
    dt = time.perf_counter() - t

    # parity spot-check of the GPU outputs on the same pairs
    def rows(off):
        sel = np.zeros((int(off[-1]), H), dtype=bool)
        for b in range(B):
            for h in range(H):
                if mask[b, h]:
                    sel[off[b]:off[b + 1], h] = True
        return sel

    def err_of(gpu, ref, sel):
        e = np.abs(gpu.float().cpu().numpy().astype(np.float64)[sel] - ref[sel])
        return {"max_abs": float(e.max()) if e.size else 0.0, "mean_abs": float(e.mean()) if e.size else 0.0,
                "elements": int(e.size)}

    selq = rows(w.q_offsets)
    parity = {"out": err_of(out_gpu, res[0], selq)}
    if with_bwd:
        selk = rows(w.k_offsets)
        for name, g, r, sel in (("dq", grads_gpu[0], res[2], selq), ("dk", grads_gpu[1], res[3], selk),
                                ("dv", grads_gpu[2], res[4], selk)):
            parity[name] = err_of(g, r, sel)
    return {"value": round(acc / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{int(mask.sum())} of {B * H} (sequence, head) pairs of the same batch, "
                      f"{'forward + backward' if with_bwd else 'forward'}, {acc:.4g} useful flop "
                      f"(same flop convention as value), fp64 C oracle on all host cores",
            "parity_on_sample": parity}


if __name__ == "__main__":
    sys.exit(main())
