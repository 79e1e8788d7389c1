"""Throughput of the selective scan (S6) forward pass on one MI355X.

One step = one sscan_forward call over the whole workload (every row of the
hot path: load/convert, ZOH discretisation, scan, readout + skip, final
state), inputs already resident in HBM.  Default workload: batch 4 x 8192
tokens x 4096 channels (Mamba-1.4B inner width), N = 16, A = -(n+1),
bf16 x/delta/B/C/y, fp32 state and arithmetic, seeded synthetic inputs.

Prints ONE JSON line: B*L*D elements/s, achieved algorithmic HBM bandwidth,
a roofline object for the scan and the fp64 oracle's throughput on a bounded
sample on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
                    [--no-cpu-baseline] [--calib-copy]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
# fp32 VALU without packed-FP32 forms: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz
# lane-ops/s; an FMA counts 2 flops -> 78.6 TFLOP/s (the published 157.3
# TFLOP/s fp32-vector figure needs the packed forms, which this build never emits).
PEAK_VALU_TFLOPS = 78.6
FLOPS_PER_UPDATE = 8           # per (b,t,d,n): 3 FMA + 2 MUL in the fused S4D-real update


def recorded_traffic(wl):
    """HBM bytes per launch of the dominant kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated with a plain copy), or None when there is no summary
    for this workload or the kernel source has changed since the counters were taken."""
    import hashlib
    import re
    prof = os.path.join(ROOT, "profiles", f"k_lockstep_{wl.name}_hbm_counters.md")
    src = os.path.join(ROOT, "selective_state_space_77_amd", "csrc", "sscan_kernels.hip")
    if not os.path.exists(prof):
        return None
    text = open(prof).read()
    m_t = re.search(r"^traffic_bytes: (\d+)$", text, re.M)
    m_h = re.search(r"^kernel_src_sha256_16: ([0-9a-f]+)$", text, re.M)
    if not (m_t and m_h):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != m_h.group(1):
        return None
    return int(m_t.group(1))


def algorithmic_bytes(wl, with_state: bool) -> int:
    es = 2 if wl.io == "bf16" else 4
    per_elem = 3 * es                                  # x, delta in; y out
    bc = 2 * wl.batch * wl.seqlen * wl.dstate * es     # B, C
    params = wl.dim * wl.dstate * 4 + wl.dim * 4       # A, Dskip
    state = wl.batch * wl.dim * wl.dstate * 4 if with_state else 0
    return wl.elements * per_elem + bc + params + state


def cpu_baseline(wl, target_s: float = 10.0) -> dict:
    """The fp64 oracle as it stands, on a prefix of the workload (whole batch rows first, then
    more rows) sized so the run takes about target_s seconds, or on the whole workload if that
    is quicker."""
    import datagen
    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    rows, T = 1, min(wl.seqlen, 256)
    while True:
        sub = datagen.Workload(wl.name, wl.key, wl.batch, wl.seqlen, wl.dim, wl.dstate, wl.io,
                               wl.a_init)
        inp = {k: datagen.gen_seq(sub, k, 0, T, batch_rows=range(rows))
               for k in ("x", "delta", "B", "C")}
        A, D = datagen.gen_A(sub), datagen.gen_Dskip(sub)
        t0 = time.perf_counter()
        oracle.forward(inp["x"], inp["delta"], A, inp["B"], inp["C"], D, nthreads=threads)
        dt = time.perf_counter() - t0
        if dt >= target_s * 0.5 or (T >= wl.seqlen and rows >= wl.batch):
            break
        grow = min(8.0, max(2.0, target_s / max(dt, 1e-3)))
        if T < wl.seqlen:
            T = min(wl.seqlen, int(T * grow))
        else:
            rows = min(wl.batch, max(rows + 1, int(rows * grow)))
    elems = rows * T * wl.dim
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"batch rows [0,{rows}), tokens [0,{T}), all {wl.dim} channels, N={wl.dstate} "
                      f"({elems} elements, {dt:.2f} s wall, fp64, {threads} threads)"}


def bench_step(wl, args, dev) -> int:
    """Decode workload: one step = one sscan_step over (batch, dim, N) fp32 state in HBM."""
    import torch

    import datagen
    import selective_state_space_77_amd as sscan

    nstage = 64  # distinct pre-staged token inputs, cycled through
    bias = datagen.gen_dt_bias(wl)
    to = lambda a: torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)
    st = [datagen.step_inputs(wl, k, bias=bias) for k in range(nstage)]
    X = torch.stack([to(s["x"]) for s in st]); Dl = torch.stack([to(s["delta"]) for s in st])
    Bs = torch.stack([to(s["B"]) for s in st]); Cs = torch.stack([to(s["C"]) for s in st])
    A = torch.from_numpy(datagen.gen_A(wl)).to(dev)
    D = torch.from_numpy(datagen.gen_Dskip(wl)).to(dev)
    state = torch.zeros(wl.batch, wl.dim, wl.dstate, device=dev)
    Y = torch.empty_like(X)
    stream = torch.cuda.current_stream(dev)
    for k in range(args.warmup):
        sscan.step(state, X[k % nstage], Dl[k % nstage], A, Bs[k % nstage], Cs[k % nstage], D,
                   y_t=Y[k % nstage], stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k, (e0, e1) in enumerate(ev):
        j = k % nstage
        e0.record(stream)
        sscan.step(state, X[j], Dl[j], A, Bs[j], Cs[j], D, y_t=Y[j], stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    per_step = (time.perf_counter() - t0) / args.steps
    ev_avg = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3
    elems = wl.batch * wl.dim
    nbytes = (2 * elems * wl.dstate * 4 + 3 * elems * 2 + 2 * wl.batch * wl.dstate * 2
              + wl.dim * wl.dstate * 4 + wl.dim * 4)
    gbs = nbytes / ev_avg / 1e9
    print(json.dumps({
        "metric": "selective-scan decode step: B*D elements/s (+ achieved HBM GB/s vs MI355X peak)",
        "value": elems / per_step, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": per_step * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded, 64 pre-staged tokens cycled)",
        "config": {"workload": wl.name, "batch": wl.batch, "dim": wl.dim, "dstate": wl.dstate,
                   "io_dtype": wl.io},
        "roofline": {"kernel": "k_step", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None,
                     "per_launch": {"algorithmic_bytes": nbytes, "event_avg_us": round(ev_avg * 1e6, 2)}},
        "cpu_baseline": None}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mamba1p4b_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy (HBM-counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan runs on a single MI355X and this build "
              "has no multi-GPU path (see the sharding note in DESIGN.md).", file=sys.stderr)
        return 2

    import torch

    import datagen
    import selective_state_space_77_amd as sscan

    wl = datagen.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if wl.mode == "step":
        return bench_step(wl, args, dev)

    # ---- inputs resident in HBM (generated per token block, seeded)
    def up(t):
        a = datagen.gen_seq(wl, t)
        if wl.io == "bf16":
            return torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    x, delta, B, C = (up(t) for t in ("x", "delta", "B", "C"))
    A = torch.from_numpy(datagen.gen_A(wl)).to(dev)
    D = torch.from_numpy(datagen.gen_Dskip(wl)).to(dev)
    y = torch.empty_like(x)
    hs = torch.empty(wl.batch, wl.dim, wl.dstate, device=dev)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] workload {wl.name}: batch={wl.batch} L={wl.seqlen} dim={wl.dim} N={wl.dstate} "
          f"io={wl.io}", file=sys.stderr, flush=True)

    def step():
        sscan.forward(x, delta, A, B, C, D, y=y, final_state=hs, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, HIP events on the launch stream around each call
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e-3  # seconds
    per_step = wall / args.steps
    ev_avg = float(durs.mean())

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    nbytes = algorithmic_bytes(wl, with_state=True)
    updates = wl.elements * wl.dstate
    hbm_gbs = nbytes / ev_avg / 1e9
    tflops = updates * FLOPS_PER_UPDATE / ev_avg / 1e12
    roof = {
        "kernel": "k_lockstep (timed: the whole sscan_forward call on its stream; the lockstep kernel is ~98% of it, the rest is the B/C staging launch and two empty-exit launches)",
        "bound": "alu",
        "achieved": round(tflops, 3),
        "peak": PEAK_VALU_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tflops / PEAK_VALU_TFLOPS, 4),
        "traffic": recorded_traffic(wl),
        "per_launch": {"updates": updates, "flops_per_update": FLOPS_PER_UPDATE,
                       "algorithmic_bytes": nbytes, "event_avg_us": round(ev_avg * 1e6, 2),
                       "event_min_us": round(float(durs.min()) * 1e6, 2)},
        "hbm": {"achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / PEAK_HBM_GBS, 4)},
    }
    out = {
        "metric": "selective-scan B*L*D elements/s (+ achieved HBM GB/s vs MI355X peak)",
        "value": wl.elements / per_step,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; x,B,C~N(0,1), delta=softplus(0.5N+bias), A=-(n+1))",
        "config": {"workload": wl.name, "batch": wl.batch, "seqlen": wl.seqlen, "dim": wl.dim,
                   "dstate": wl.dstate, "io_dtype": wl.io, "a_init": wl.a_init},
        "hbm_gbs": round(nbytes / per_step / 1e9, 1),
        "hbm_frac_of_peak": round(nbytes / per_step / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(wl),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
