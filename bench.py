#!/usr/bin/env python3
"""Throughput of the jagged attention hot path on one MI355X; prints ONE JSON line.

A step is one full ``jagged_attn_fwd`` call (device tile scheduler + fused attention
kernel) over the whole synthetic batch, inputs already resident in HBM. The default
workload is the jagged causal softmax self-attention batch (B=64, lengths
log-uniform in [128, 4096], H=4, d=128, bf16). ``--workload 3|4|5|6`` measures the
other named batches (6: 64-token block-diagonal attention through
``jagged_block_attn_fwd``; 7: QK-normed self-attention with the ALU-only GELU);
``--bwd`` adds the backward (softmax for 2, 5 and 6, the pointwise SiLU / GELU
backward for 3, 4 and 7); ``--act`` swaps the activation.

Before the warm-up steps the step runs untimed for --spinup-ms (default 200 ms): an
idle GPU takes tens of milliseconds of load to reach its working clock, which five
warm-up steps of a fraction of a millisecond do not give it.

Reported:
  value        useful (unpadded) TFLOP/s of the whole step: 4 d H sum_b pairs_b per
               forward (10 d H pairs for the backward), pairs_b = visible (query,
               key) pairs of sequence b, over the measured step time;
  roofline     the forward attention kernel alone, timed with HIP events recorded on
               its own stream right before and after its launch (library profiling
               hook): useful TFLOP/s against the published dense bf16 MFMA peak, or,
               for the HBM-bound batches (3, 4, 6), algorithmic bytes (Q, K, V read
               and O written once) per second against the published 8 TB/s;
               `traffic` is HBM bytes per launch from committed rocprofv3 counter
               runs, or null when the kernel source changed since they were taken;
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
HBM_BOUND = (3, 4, 6)         # workloads whose forward is bound by HBM traffic, not the matrix cores
KERNEL_SOURCES = {
    "ja_fwd_kernel": ["ja_fwd.hip", "ja_common.h", "ja_lds.h", "ja_tiles.h", "ja_internal.h"],
    "ja_mx_fwd_kernel": ["ja_mx.hip", "ja_mx.h", "ja_common.h", "ja_lds.h", "ja_tiles.h", "ja_internal.h"],
    "ja_bwd_kernels": ["ja_bwd.hip", "ja_common.h", "ja_lds.h", "ja_tiles.h", "ja_internal.h"],
}
METRIC = "useful (unpadded) bf16 TFLOP/s of jagged attn fwd; % of MI355X MFMA peak"


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


def roofline_kernel(workload: int) -> str:
    """The kernel the roofline is taken on: the forward attention kernel (the MXFP8
    forward for workload 8; every other workload, the block one included, runs the
    general forward)."""
    return "ja_mx_fwd_kernel" if workload == 8 else "ja_fwd_kernel"


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5, 6, 7, 8])
    ap.add_argument("--bwd", action="store_true",
                    help="time forward + backward (softmax for 2, 5 and 6, SiLU / GELU for 3, 4 and 7)")
    ap.add_argument("--act", choices=["softmax", "silu", "gelu", "gelu_taylor"], default=None,
                    help="run the workload with another activation (e.g. 7 with the tanh GELU)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle budget for the CPU baseline")
    ap.add_argument("--spinup-ms", type=float, default=200.0,
                    help="untimed load before the warm-up steps, so the GPU has left its idle clock state")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy (y = x * 1) of MIB MiB, 5 times: the reference "
                         "for scaling HBM byte counters")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="no GPU: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of --workload (and of "
                         "--copy-calibration 1024) into HBM bytes per forward launch in profiles/traffic.json")
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

    log(f"[bench] generating workload {args.workload}")
    w = W.workload(args.workload, act=args.act)
    if args.bwd and w.dout is None:
        W.with_upstream_gradient(w, 1000 + args.workload)  # seeded dO for the batches that draw none

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        return t.to(dev)

    q, k, v = up(w.q), up(w.k), up(w.v)
    qo, ko = up(w.q_offsets), up(w.k_offsets)
    dout = up(w.dout) if args.bwd else None
    mx = bool(w.extra.get("mxfp8"))
    if mx:
        if args.bwd:
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
    need_lse = w.act == "softmax" and not (w.block and w.block <= 64)
    lse = torch.empty((Tq, w.H), dtype=torch.float32, device=dev) if need_lse else None
    if mx:
        ws_fwd, ws_bwd = int(lib.ja_fwd_mxfp8_workspace_size(w.B, w.H, w.d, Tq, Tk)), 0
    elif w.block:
        ws_fwd = ws_bwd = ja.block_attn_workspace_size(w.B, w.H, w.d, Tq, w.block, w.causal)
    else:
        ws_fwd = ja.fwd_workspace_size(w.B, w.H, w.d, Tq, Tk, w.act, w.causal, w.window)
        ws_bwd = ja.bwd_workspace_size(w.B, w.H, w.d, Tq, Tk, w.act, w.causal, w.window) if args.bwd else 0
    ws = torch.empty(max(ws_fwd, 256), dtype=torch.uint8, device=dev)
    if args.bwd:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(max(ws_bwd, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    pairs = visible_pairs(w.lq, w.lk, w.causal, w.window, w.block)
    fwd_flop = 4.0 * w.d * w.H * pairs
    bwd_flop = 10.0 * w.d * w.H * pairs if args.bwd else 0.0

    def step(ev=None):
        if ev is not None:
            lib.ja_set_profile_events(ev[0].cuda_event, ev[1].cuda_event)
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
        if args.bwd:
            if ev is not None:
                lib.ja_set_profile_events(ev[2].cuda_event, ev[3].cuda_event)
            if w.block:
                ja.jagged_block_attn_bwd(q, k, v, out, dout, lse, qo, w.block, causal=w.causal, scale=w.scale,
                                         dq=dq, dk=dk, dv=dv, workspace=bws, stream=stream)
            else:
                ja.jagged_attn_bwd(q, k, v, out, dout, lse, qo, ko, act=w.act, causal=w.causal, window=w.window,
                                   scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=bws, stream=stream)
        if ev is not None:
            lib.ja_set_profile_events(None, None)

    # An idle GPU needs tens of milliseconds of load to reach its working clock (on
    # MI355X the w2 forward measures 0.205 ms after 5 warm-up steps, 0.178 ms after
    # 200): run the same step, untimed, for spinup_ms before the warm-up steps.
    log(f"[bench] spin-up {args.spinup_ms:.0f} ms, then warmup {args.warmup} steps")
    t_end = time.perf_counter() + args.spinup_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    nev = 4 if args.bwd else 2
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for evs in events:  # create the underlying HIP events before handing them to the library
        for e in evs:
            e.record(stream)
    whole0, whole1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    whole0.record(stream)
    for i in range(args.steps):
        step(events[i])
    whole1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ms_events = whole0.elapsed_time(whole1) / args.steps
    fwd_kernel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    bwd_kernel_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events])) if args.bwd else None
    total_flop = fwd_flop + bwd_flop
    value = total_flop / (ms_per_step * 1e-3) / 1e12

    name = roofline_kernel(args.workload)
    tflops = fwd_flop / (fwd_kernel_ms * 1e-3) / 1e12
    if args.workload in HBM_BOUND:
        # short key/value (3), short query (4) and 64-token block (6) batches are
        # HBM-bound: the algorithmic traffic is reading Q, K, V once and writing O
        # (and the fp32 lse where the backward needs it) once.
        min_bytes = 2 * w.H * w.d * (2 * Tq + 2 * Tk) + (4 * w.H * Tq if need_lse else 0)
        gbs = min_bytes / (fwd_kernel_ms * 1e-3) / 1e9
        copy = measure_copy_gbs(1024)  # what a plain streaming kernel sustains on this GPU, same run
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": min_bytes,
                    "copy_gbs": round(copy, 1), "frac_of_copy": round(gbs / copy, 4),
                    "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    else:
        peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tflops / peak, 4), "flop_per_launch": fwd_flop}
    roofline["traffic"] = recorded_traffic(name, f"w{args.workload}")
    roofline["kernel"] = name
    roofline["kernel_ms"] = round(fwd_kernel_ms, 4)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spinup_ms": args.spinup_ms,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_events": round(ms_events, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "pct_of_peak": round(100.0 * value / (PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS), 2),
        "dtype": "fp8-e4m3 (MX, [32,32] block scales)" if mx else "bf16",
        "data": "synthetic",
        "config": {"workload": w.extra.get("description", w.name), "B": w.B, "H": w.H, "d": w.d,
                   "act": w.act, "causal": bool(w.causal), "window": int(w.window), "block": int(w.block),
                   "scale": round(w.scale, 6),
                   "q_tokens": int(Tq),
                   "kv_tokens": int(Tk), "visible_pairs": int(pairs), "fwd_flop": fwd_flop,
                   "bwd_flop": bwd_flop, "phases": "fwd+bwd" if args.bwd else "fwd"},
        "roofline": roofline,
    }
    if args.bwd:
        result["bwd"] = {"kernel_ms": round(bwd_kernel_ms, 4),
                         "tflops": round(bwd_flop / (bwd_kernel_ms * 1e-3) / 1e12, 2)}
        if args.workload in (3, 4, 6):
            # reading Q, K, V, dO once and writing dQ, dK, dV once (the two-pass
            # softmax backward also reads O and lse)
            min_b = 2 * w.H * w.d * (3 * Tq + 4 * Tk)
            if need_lse:
                min_b += 2 * w.H * w.d * Tq + 4 * w.H * Tq
            result["bwd"]["min_hbm_bytes"] = min_b
            result["bwd"]["hbm_gbs_at_min_bytes"] = round(min_b / (bwd_kernel_ms * 1e-3) / 1e9, 1)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, out, lse, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


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


def record_traffic(workload: int, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str) -> int:
    """HBM bytes per forward launch = FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled so that the copy kernel of known size reads and writes exactly its bytes."""
    copy_bytes = 1024 * (1 << 20)
    cf = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "elementwise")
    cw = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "elementwise")
    name = roofline_kernel(workload)
    kf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", name)
    kw = _counter_per_dispatch(write_dir, "WRITE_SIZE", name)
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
    data.setdefault(name, {})[f"w{workload}"] = {
        "hbm_bytes_per_launch": round(fetch + write),
        "fetch_bytes": round(fetch), "write_bytes": round(write),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "source_sha256": kernel_sha(name),
        "method": "rocprofv3 --pmc FETCH_SIZE then --pmc WRITE_SIZE on bench.py --workload "
                  f"{workload} --steps 2 --warmup 1 --no-cpu-baseline; KiB per dispatch (median) x 1024 x "
                  "scale, scale = 1 GiB / the same counter on bench.py --copy-calibration 1024",
    }
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(data[name][f"w{workload}"]))
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


def cpu_baseline(w, out_gpu, lse_gpu, budget_s: float) -> dict:
    """Time the fp64 oracle on a bounded sample of (sequence, head) pairs of the batch."""
    import oracle  # test infrastructure: used here for the CPU baseline only

    if w.extra.get("mxfp8"):
        # the MXFP8 forward on the oracle's quantization of the batch (bit-identical to
        # the library's, which the tests check); the quantization itself is upstream
        qm = oracle.mxfp8_quantize(w.q, w.q_offsets)
        km = oracle.mxfp8_quantize(w.k, w.k_offsets)
        vm = oracle.mxfp8_quantize(w.v, w.k_offsets)

        def run_oracle(mask):
            return oracle.fwd_mxfp8(qm[0], qm[1], qm[2], km[0], km[1], km[2], vm[0], vm[1], w.q_offsets,
                                    w.k_offsets, w.causal, w.window, w.scale, pquant=True, pair_mask=mask)
    else:
        def run_oracle(mask):
            return oracle.fwd(w.q, w.k, w.v, w.q_offsets, w.k_offsets, w.act, w.causal, w.window, w.scale,
                              pair_mask=mask, block=w.block)

    rng = np.random.default_rng(1234)
    B, H = w.B, w.H
    order = [(int(b), int(h)) for b in rng.permutation(B) for h in range(H)]
    pair_flop = np.array([4.0 * w.d * visible_pairs(w.lq[b:b + 1], w.lk[b:b + 1], w.causal, w.window, w.block)
                          for b, _ in order])
    # Calibrate the oracle's rate on a growing prefix of the pair order (at least
    # ~1 s of work), then fill the budget.
    mask = np.zeros((B, H), dtype=bool)
    rate, n_cal = None, 1
    while rate is None:
        mask[:] = False
        for b, h in order[:n_cal]:
            mask[b, h] = True
        t = time.perf_counter()
        run_oracle(mask)
        dt = time.perf_counter() - t
        if dt >= 1.0 or n_cal >= len(order):
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
    ref, ref_lse = run_oracle(mask)
    dt = time.perf_counter() - t
    # parity spot-check of the GPU output on the same pairs
    got = out_gpu.float().cpu().numpy().astype(np.float64)
    sel = np.zeros(got.shape[:2], dtype=bool)
    for b in range(B):
        for h in range(H):
            if mask[b, h]:
                sel[w.q_offsets[b]:w.q_offsets[b + 1], h] = True
    err = np.abs(got[sel] - ref[sel])
    return {"value": round(acc / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{int(mask.sum())} of {B * H} (sequence, head) pairs of the same batch, "
                      f"{acc:.4g} useful flop, fp64 C oracle on all host cores",
            "parity_on_sample": {"max_abs": float(err.max()) if err.size else 0.0,
                                 "mean_abs": float(err.mean()) if err.size else 0.0,
                                 "elements": int(err.size)}}


if __name__ == "__main__":
    sys.exit(main())
