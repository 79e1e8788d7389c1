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
                    [--pass forward|backward] [--no-cpu-baseline] [--calib-copy]

--pass backward times sscan_backward instead (all seven gradients, the same
workload, dy and dfinal_state seeded like x); --pass fused times
sscan_forward_fused (d_conv = 4, SiLU, carried inputs and biases) on the same
workload, x being the convolution's raw input and delta the raw step size.
--workload decode_bf16 times sscan_step, --workload mamba2_bf16 sscan_ssd_forward and
--workload mamba2_decode_bf16 sscan_ssd_step (the scalar-A-per-head scan and its step).
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
# TFLOP/s fp32-vector figure needs the packed forms, which this library never emits).
PEAK_VALU_TFLOPS = 78.6
FLOPS_PER_UPDATE = 8           # per (b,t,d,n): 4 FMA: w - k, the state update, the 1 - Abar recurrence, the readout
# backward, per (b,t,d,n): the recomputed forward update (8) plus the adjoint and
# gradient terms, each an FMA (2) or a multiply (1): lam = C*dy + carry (2),
# lam*gain (1), dx += .*B (2), B*x (1), A*h_t + Bx (2), ddelta += lam*. (2),
# delta*Abar (1), .*h_{t-1} + dgain/dA*Bx (3), dA += lam*. (2), dB term lam*gain*x (1),
# dC term dy*h_t (1), carry Abar*lam (1)
FLOPS_PER_UPDATE_BWD = 8 + 19
# fused front end, per (b,t,d) element: 4 conv taps + bias (8), SiLU (exp, add, reciprocal,
# multiply: 4), softplus of the biased raw step (add, exp, add, log, multiply, max: 6)
FLOPS_PER_ELEMENT_FE = 18
D_CONV = 4
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak, published


CSRC = os.path.join(ROOT, "selective_state_space_77_amd", "csrc")
FWD_SOURCES = ("sscan_kernels.hip", "sscan_device.h", "sscan_internal.h")
BWD_SOURCES = ("sscan_bwd.hip", "sscan_device.h", "sscan_internal.h")
SSD_SOURCES = ("sscan_ssd.hip", "sscan_device.h", "sscan_internal.h")


def source_fingerprint(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(summary: str, sources):
    """HBM bytes per launch of the dominant kernel from a committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated with a plain copy), or None when the summary is
    missing or the kernel sources have changed since the counters were taken."""
    import re
    prof = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(prof):
        return None
    text = open(prof).read()
    m_t = re.search(r"^traffic_bytes: (\d+)$", text, re.M)
    m_h = re.search(r"^kernel_src_sha256_16: ([0-9a-f]+)$", text, re.M)
    if not (m_t and m_h) or source_fingerprint(sources) != m_h.group(1):
        return None
    return int(m_t.group(1))


def recorded_value(summary: str, key: str, sources):
    """A figure ("key: value" line) from a committed counter summary, or None when the
    summary is missing or the kernel sources have changed since it was taken."""
    import re
    prof = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(prof):
        return None
    text = open(prof).read()
    m_v = re.search(rf"^{re.escape(key)}: ([0-9.eE+-]+)$", text, re.M)
    m_h = re.search(r"^kernel_src_sha256_16: ([0-9a-f]+)$", text, re.M)
    if not (m_v and m_h) or source_fingerprint(sources) != m_h.group(1):
        return None
    return float(m_v.group(1))


def cpu_info() -> dict:
    """The host CPU the oracle baseline runs on: model name and the cores this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return {"model": model, "logical_cpus": os.cpu_count(), "available_cpus": avail}


FLUSH_BYTES = 512 << 20  # written between cold runs: more than L2 and the 256 MB Infinity Cache
COLD_RUNS = 20


def _cold_median(call, stream, dev, runs: int = COLD_RUNS):
    """Median (and min) event time of `runs` calls, each preceded on the same stream by a
    FLUSH_BYTES write that evicts the caches, so every call starts from HBM."""
    import torch
    buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    with torch.cuda.stream(stream):
        for i, (e0, e1) in enumerate(ev):
            buf.fill_(float(i))
            e0.record(stream)
            call()
            e1.record(stream)
    torch.cuda.synchronize()
    d = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e-3
    del buf
    return float(np.median(d)), float(d.min())


def copy_bandwidth(dev, nbytes: int = 1 << 30, runs: int = 10) -> float:
    """Achievable HBM bandwidth on this device: a plain nbytes device-to-device copy,
    (read + write bytes) / median event time, in GB/s."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for e0, e1 in ev:
        e0.record()
        dst.copy_(src)
        e1.record()
    torch.cuda.synchronize()
    t = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3
    del src, dst
    return 2 * nbytes / t / 1e9


def algorithmic_bytes(wl, with_state: bool) -> int:
    es = 2 if wl.io == "bf16" else 4
    per_elem = 3 * es                                  # x, delta in; y out
    bc = 2 * wl.batch * wl.seqlen * wl.dstate * es     # B, C
    params = wl.dim * wl.dstate * 4 + wl.dim * 4       # A, Dskip
    state = wl.batch * wl.dim * wl.dstate * 4 if with_state else 0
    return wl.elements * per_elem + bc + params + state


def _oracle_rate(wl, threads: int, target_s: float):
    """The oracle's forward on a prefix of the workload (whole batch rows first, then more
    rows) sized to about target_s, or on the whole workload when that is quicker.
    Returns (elements/s, rows, tokens, seconds)."""
    import datagen
    import oracle

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
    return rows * T * wl.dim / dt, rows, T, dt


def cpu_baseline(wl, target_s: float = 10.0) -> dict:
    """The fp64 oracle as it stands, on the host cores: every core this process may use
    (16 at most: the share of one GPU's host) on a bounded prefix of the benchmarked
    workload, and one thread on a prefix of the 8 x 2048 x 1536 fp32 workload."""
    import datagen

    info = cpu_info()
    threads = max(1, min(16, info["available_cpus"]))
    v, rows, T, dt = _oracle_rate(wl, threads, target_s)
    v1, rows1, T1, dt1 = _oracle_rate(datagen.workload("mamba130m_f32"), 1, target_s / 2)
    return {"value": v, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"batch rows [0,{rows}), tokens [0,{T}), all {wl.dim} channels, N={wl.dstate} "
                      f"({rows * T * wl.dim} elements, {dt:.2f} s wall, fp64, {threads} threads)",
            "cpu_model": info["model"], "logical_cpus": info["logical_cpus"],
            "single_thread": {"value": v1, "unit": "elements/s", "cores": 1,
                              "sample": f"mamba130m_f32: batch rows [0,{rows1}), tokens [0,{T1}), "
                                        f"all 1536 channels, N=16 ({dt1:.2f} s wall)"}}


def _calib_copy(dev):
    """A plain 1 GiB device copy: the reference point for the HBM byte counters."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def _upload(wl, t, dev):
    import torch

    import datagen
    a = datagen.gen_seq(wl, t)
    if wl.io == "bf16":
        return torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def _time(call, steps, warmup, stream):
    """W untimed calls, then exactly K timed calls back to back, between one pair of HIP
    events on the launch stream and a synchronisation on each side.  (The GPU's clock ramps
    up over its first tens of milliseconds of work, which is what the warmup covers; events
    recorded around every call slowed the calls by about 3%, so there are none in between.)
    Returns (wall seconds per call, event seconds per call)."""
    import torch
    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    return wall, e0.elapsed_time(e1) * 1e-3 / steps


def cpu_baseline_backward(wl, target_s: float = 10.0) -> dict:
    """The oracle's backward pass on a token prefix of batch row 0, sized to about target_s."""
    import datagen
    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    T = min(wl.seqlen, 64)
    while True:
        inp = {k: datagen.gen_seq(wl, k, 0, T, batch_rows=[0]) for k in ("x", "delta", "B", "C", "dy")}
        A, D = datagen.gen_A(wl), datagen.gen_Dskip(wl)
        t0 = time.perf_counter()
        oracle.backward(inp["x"], inp["delta"], A, inp["B"], inp["C"], D, inp["dy"], nthreads=threads)
        dt = time.perf_counter() - t0
        if dt >= target_s * 0.5 or T >= wl.seqlen:
            break
        T = min(wl.seqlen, int(T * min(8.0, max(2.0, target_s / max(dt, 1e-3)))))
    elems = T * wl.dim
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"backward, batch row 0, tokens [0,{T}), all {wl.dim} channels, N={wl.dstate} "
                      f"({elems} elements, {dt:.2f} s wall, fp64, {threads} threads)"}


def bench_backward(wl, args, dev) -> int:
    """One step = one sscan_backward call over the whole workload (recomputed states, all
    gradients), inputs and cotangents resident in HBM."""
    import torch

    import datagen
    import selective_state_space_77_amd as sscan

    x, delta, B, C, dy = (_upload(wl, t, dev) for t in ("x", "delta", "B", "C", "dy"))
    A = torch.from_numpy(datagen.gen_A(wl)).to(dev)
    D = torch.from_numpy(datagen.gen_Dskip(wl)).to(dev)
    dhT = torch.from_numpy(datagen.gen_state(wl, "dhT")).to(dev)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] backward {wl.name}: batch={wl.batch} L={wl.seqlen} dim={wl.dim} N={wl.dstate} "
          f"io={wl.io}", file=sys.stderr, flush=True)
    wall, ev_avg = _time(
        lambda: sscan.backward(x, delta, A, B, C, dy, Dskip=D, dfinal_state=dhT, stream=stream),
        args.steps, args.warmup, stream)
    if args.calib_copy:
        _calib_copy(dev)
    es = 2 if wl.io == "bf16" else 4
    nbytes = (wl.elements * 5 * es                                  # x, delta, dy in; dx, ddelta out
              + wl.batch * wl.seqlen * wl.dstate * (2 * es + 2 * 4)  # B, C in; dB, dC (fp32) out
              + 2 * (wl.dim * wl.dstate * 4 + wl.dim * 4)           # A, Dskip in; dA, dDskip out
              + 2 * wl.batch * wl.dim * wl.dstate * 4)              # dfinal_state in, dinitial_state out
    updates = wl.elements * wl.dstate
    tflops = updates * FLOPS_PER_UPDATE_BWD / ev_avg / 1e12
    gbs = nbytes / ev_avg / 1e9
    print(json.dumps({
        "metric": "selective-scan backward: B*L*D elements/s",
        "value": wl.elements / wall, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; x,B,C,dy~N(0,1), delta=softplus(0.5N+bias))",
        "config": {"workload": wl.name, "pass": "backward", "batch": wl.batch, "seqlen": wl.seqlen,
                   "dim": wl.dim, "dstate": wl.dstate, "io_dtype": wl.io, "a_init": wl.a_init},
        "roofline": {"kernel": "k_bwd_ckpt + k_bwd + k_bwd_reduce (timed: the whole sscan_backward "
                                "call on its stream; k_bwd, the reverse pass, is ~90% of it)",
                     "bound": "alu", "achieved": round(tflops, 3), "peak": PEAK_VALU_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_VALU_TFLOPS, 4),
                     "traffic": recorded_traffic(f"k_bwd_{wl.name}_hbm_counters.md", BWD_SOURCES),
                     "per_launch": {"updates": updates, "flops_per_update": FLOPS_PER_UPDATE_BWD,
                                    "algorithmic_bytes": nbytes,
                                    "event_avg_us": round(ev_avg * 1e6, 2)},
                     "hbm": {"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4)}},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_backward(wl)}), flush=True)
    return 0


def bench_fused(wl, args, dev) -> int:
    """One step = one sscan_forward_fused call: the causal convolution (d_conv = 4, SiLU) of x
    and softplus(delta_raw + bias) formed inside the scan kernels, then the scan."""
    import torch

    import datagen
    import selective_state_space_77_amd as sscan

    fe = datagen.frontend_inputs(wl, D_CONV)
    x, B, C = (_upload(wl, t, dev) for t in ("x", "B", "C"))
    to = (lambda a: torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)) \
        if wl.io == "bf16" else (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev))
    draw, cs = to(fe["delta_raw"]), to(fe["conv_state"])
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    cw, cb, db = f32(fe["conv_w"]), f32(fe["conv_b"]), f32(fe["delta_bias"])
    A = torch.from_numpy(datagen.gen_A(wl)).to(dev)
    D = torch.from_numpy(datagen.gen_Dskip(wl)).to(dev)
    y = torch.empty_like(x)
    hs = torch.empty(wl.batch, wl.dim, wl.dstate, device=dev)
    cso = torch.empty_like(cs)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] fused {wl.name}: batch={wl.batch} L={wl.seqlen} dim={wl.dim} N={wl.dstate} "
          f"io={wl.io} d_conv={D_CONV} silu", file=sys.stderr, flush=True)
    wall, ev_avg = _time(
        lambda: sscan.forward_fused(x, cw, draw, A, B, C, D, conv_bias=cb, delta_bias=db,
                                    activation="silu", conv_state=cs, y=y, final_state=hs,
                                    conv_state_out=cso, stream=stream),
        args.steps, args.warmup, stream)
    if args.calib_copy:
        _calib_copy(dev)
    nbytes = algorithmic_bytes(wl, with_state=True) + wl.dim * (D_CONV + 2) * 4 \
        + 2 * wl.batch * (D_CONV - 1) * wl.dim * (2 if wl.io == "bf16" else 4)
    updates = wl.elements * wl.dstate
    flops = updates * FLOPS_PER_UPDATE + wl.elements * FLOPS_PER_ELEMENT_FE
    tflops = flops / ev_avg / 1e12
    gbs = nbytes / ev_avg / 1e9
    print(json.dumps({
        "metric": "selective-scan with fused front end: B*L*D elements/s",
        "value": wl.elements / wall, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; x,B,C~N(0,1), delta_raw=0.5N, conv taps U(+-1/2))",
        "config": {"workload": wl.name, "pass": "fused", "d_conv": D_CONV, "activation": "silu",
                   "batch": wl.batch, "seqlen": wl.seqlen, "dim": wl.dim, "dstate": wl.dstate,
                   "io_dtype": wl.io, "a_init": wl.a_init},
        "roofline": {"kernel": "k_lockstep<.., FE> (timed: the whole sscan_forward_fused call)",
                     "bound": "alu", "achieved": round(tflops, 3), "peak": PEAK_VALU_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_VALU_TFLOPS, 4),
                     "traffic": recorded_traffic(f"k_lockstep_fused_{wl.name}_hbm_counters.md", FWD_SOURCES),
                     "per_launch": {"updates": updates, "flops": flops, "algorithmic_bytes": nbytes,
                                    "event_avg_us": round(ev_avg * 1e6, 2)},
                     "hbm": {"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4)}},
        "cpu_baseline": None}), flush=True)
    return 0


def bench_ssd(wl, args, dev) -> int:
    """Scalar-A-per-head scan (Mamba-2 shape): one step = one sscan_ssd_forward over the whole
    workload (chunked matrix form, products on the matrix cores), inputs resident in HBM."""
    import torch

    import datagen
    import selective_state_space_77_amd as sscan

    inp = datagen.ssd_inputs(wl)
    to = (lambda a: torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)) \
        if wl.io == "bf16" else (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev))
    x, delta, B, C = (to(inp[k]) for k in ("x", "delta", "B", "C"))
    A, D = torch.from_numpy(inp["A"]).to(dev), torch.from_numpy(inp["D"]).to(dev)
    y = torch.empty_like(x)
    hs = torch.empty(wl.batch, wl.nheads, wl.headdim, wl.dstate, device=dev)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] ssd {wl.name}: batch={wl.batch} L={wl.seqlen} heads={wl.nheads} P={wl.headdim} "
          f"groups={wl.ngroups} N={wl.dstate} io={wl.io}", file=sys.stderr, flush=True)
    wall, ev_avg = _time(
        lambda: sscan.ssd_forward(x, delta, A, B, C, D, y=y, final_state=hs, stream=stream),
        args.steps, args.warmup, stream)
    if args.calib_copy:
        _calib_copy(dev)
    es = 2 if wl.io == "bf16" else 4
    BL = wl.batch * wl.seqlen
    nbytes = (2 * wl.elements * es + BL * wl.nheads * es + 2 * BL * wl.ngroups * wl.dstate * es
              + 2 * wl.nheads * 4 + wl.batch * wl.nheads * wl.headdim * wl.dstate * 4)
    # algorithmic matrix flops per (token, head) of the chunked form with 64-token chunks:
    # scores C B^T over the causal half (incl. diagonal), scores x X, C S_in, B^T (w X)
    Q = 64
    per_tok = 2 * (Q + 1) / 2 * (wl.dstate + wl.headdim) + 2 * 2 * wl.dstate * wl.headdim
    flops = per_tok * BL * wl.nheads
    gbs = nbytes / ev_avg / 1e9
    tflops = flops / ev_avg / 1e12
    print(json.dumps({
        "metric": "scalar-A-per-head scan (Mamba-2 SSM): B*L*H*P elements/s",
        "value": wl.elements / wall, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.io == "bf16" else "f32",
        "data": "synthetic (seeded; x,B,C~N(0,1), delta=softplus(0.5N+bias), A=-exp(U(0,log16)))",
        "config": {"workload": wl.name, "batch": wl.batch, "seqlen": wl.seqlen, "nheads": wl.nheads,
                   "headdim": wl.headdim, "ngroups": wl.ngroups, "dstate": wl.dstate, "io_dtype": wl.io},
        "roofline": {"kernel": "k_ssd_bf" if wl.io == "bf16" else "k_ssd", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic(f"k_ssd_{wl.name}_hbm_counters.md", SSD_SOURCES),
                     "per_launch": {"algorithmic_bytes": nbytes, "matrix_flops": flops,
                                    "event_avg_us": round(ev_avg * 1e6, 2)},
                     "mfma": {"achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}},
        "cpu_baseline": None}), flush=True)
    return 0


def bench_step(wl, args, dev) -> int:
    """Decode workload: one bench step = the workload's wl.seqlen (1000) consecutive sscan_step
    calls on the (batch, dim, N) fp32 state in HBM, every token's inputs pre-staged on the
    device.  The 84 MB state stays in the 256 MB Infinity Cache from one call to the next, so
    the per-call rate is also measured with the state rotated over four buffers (336 MB)."""
    import torch
    from concurrent.futures import ThreadPoolExecutor

    import datagen
    import selective_state_space_77_amd as sscan

    S = wl.seqlen
    bias = datagen.gen_dt_bias(wl)
    to = lambda a: torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)
    X = torch.empty(S, wl.batch, wl.dim, dtype=torch.bfloat16, device=dev)
    Dl = torch.empty_like(X)
    Bs = torch.empty(S, wl.batch, wl.dstate, dtype=torch.bfloat16, device=dev)
    Cs = torch.empty_like(Bs)
    print(f"[bench] decode {wl.name}: staging {S} steps of {wl.batch}x{wl.dim}", file=sys.stderr, flush=True)
    with ThreadPoolExecutor(max(1, min(16, cpu_info()["available_cpus"]))) as ex:
        for k, st in ex.map(lambda k: (k, datagen.step_inputs(wl, k, bias=bias)), range(S)):
            X[k], Dl[k], Bs[k], Cs[k] = to(st["x"]), to(st["delta"]), to(st["B"]), to(st["C"])
    A = torch.from_numpy(datagen.gen_A(wl)).to(dev)
    D = torch.from_numpy(datagen.gen_Dskip(wl)).to(dev)
    states = [torch.zeros(wl.batch, wl.dim, wl.dstate, device=dev) for _ in range(4)]
    Y = torch.empty_like(X)
    stream = torch.cuda.current_stream(dev)

    def run(rotate: bool):
        for k in range(S):
            sscan.step(states[k % 4 if rotate else 0], X[k], Dl[k], A, Bs[k], Cs[k], D, y_t=Y[k], stream=stream)

    wall, ev_avg = _time(lambda: run(False), args.steps, args.warmup, stream)
    _, rot_avg = _time(lambda: run(True), max(1, args.steps // 4), 1, stream)
    copy_gbs = copy_bandwidth(dev)
    per_call = ev_avg / S
    elems = wl.batch * wl.dim
    nbytes = (2 * elems * wl.dstate * 4 + 3 * elems * 2 + 2 * wl.batch * wl.dstate * 2
              + wl.dim * wl.dstate * 4 + wl.dim * 4)
    gbs = nbytes / per_call / 1e9
    rot_gbs = nbytes / (rot_avg / S) / 1e9
    print(json.dumps({
        "metric": "selective-scan decode step: B*D elements/s (+ achieved HBM GB/s vs MI355X peak)",
        "value": S * elems / wall, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": f"synthetic (seeded; one step = {S} consecutive decode steps, every token's inputs "
                f"pre-staged in HBM)",
        "config": {"workload": wl.name, "batch": wl.batch, "dim": wl.dim, "dstate": wl.dstate,
                   "io_dtype": wl.io, "decode_steps_per_step": S},
        "copy_gbs": round(copy_gbs, 1),
        "roofline": {"kernel": "k_step", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "note": "the 84 MB state stays in the 256 MB Infinity Cache between calls: "
                             "achieved counts algorithmic bytes over fabric; state_rotated is the rate "
                             "with four state buffers (336 MB) used in turn",
                     "traffic": recorded_traffic(f"k_step_{wl.name}_hbm_counters.md", FWD_SOURCES),
                     "per_launch": {"algorithmic_bytes": nbytes, "event_avg_us": round(per_call * 1e6, 2)},
                     "state_rotated": {"achieved": round(rot_gbs, 1), "frac": round(rot_gbs / PEAK_HBM_GBS, 4),
                                       "event_avg_us": round(rot_avg / S * 1e6, 2)}},
        "cpu_baseline": None}), flush=True)
    return 0


def bench_ssd_step(wl, args, dev) -> int:
    """Scalar-A-per-head decode: one step = one sscan_ssd_step over the (batch, heads, 64, N)
    fp32 state in HBM, token inputs cycled through wl.seqlen pre-staged ones."""
    import torch

    import datagen
    import selective_state_space_77_amd as sscan

    inp = datagen.ssd_inputs(wl)
    to = (lambda a: torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)) \
        if wl.io == "bf16" else (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev))
    # token-major staging: step k reads row k of each
    X, Dl, Bs, Cs = (to(np.ascontiguousarray(np.moveaxis(inp[k], 1, 0))) for k in ("x", "delta", "B", "C"))
    A, D = torch.from_numpy(inp["A"]).to(dev), torch.from_numpy(inp["D"]).to(dev)
    state = torch.zeros(wl.batch, wl.nheads, wl.headdim, wl.dstate, device=dev)
    Y = torch.empty_like(X)
    nstage = wl.seqlen
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] ssd decode {wl.name}: batch={wl.batch} heads={wl.nheads} P={wl.headdim} "
          f"groups={wl.ngroups} N={wl.dstate} io={wl.io}", file=sys.stderr, flush=True)
    count = [0]

    def one():  # the next staged token's inputs
        j = count[0] % nstage
        count[0] += 1
        sscan.ssd_step(state, X[j], Dl[j], A, Bs[j], Cs[j], D, y_t=Y[j], stream=stream)

    per_step, ev_avg = _time(one, args.steps, args.warmup, stream)
    es = 2 if wl.io == "bf16" else 4
    chans = wl.batch * wl.nheads * wl.headdim
    nbytes = (2 * chans * wl.dstate * 4 + 2 * chans * es + wl.batch * wl.nheads * es
              + 2 * wl.batch * wl.ngroups * wl.dstate * es + 2 * wl.nheads * 4)
    gbs = nbytes / ev_avg / 1e9
    print(json.dumps({
        "metric": "scalar-A-per-head decode step: B*H*P elements/s (+ achieved HBM GB/s vs MI355X peak)",
        "value": chans / per_step, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": per_step * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": f"synthetic (seeded, {nstage} pre-staged tokens cycled)",
        "config": {"workload": wl.name, "batch": wl.batch, "nheads": wl.nheads, "headdim": wl.headdim,
                   "ngroups": wl.ngroups, "dstate": wl.dstate, "io_dtype": wl.io},
        "roofline": {"kernel": "k_ssd_step", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic(f"k_ssd_step_{wl.name}_hbm_counters.md", SSD_SOURCES),
                     "per_launch": {"algorithmic_bytes": nbytes, "event_avg_us": round(ev_avg * 1e6, 2)}},
        "cpu_baseline": None}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first: the GPU's clock ramps up over its first tens of ms of work")
    ap.add_argument("--workload", default="mamba1p4b_bf16")
    ap.add_argument("--pass", dest="which", choices=("forward", "backward", "fused"), default="forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy (HBM-counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan runs on a single MI355X and the library "
              "has no multi-GPU path.", file=sys.stderr)
        return 2

    import torch

    import datagen
    import selective_state_space_77_amd as sscan

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in datagen.SSD_WORKLOADS:
        swl = datagen.SSD_WORKLOADS[args.workload]
        return (bench_ssd_step if swl.mode == "step" else bench_ssd)(swl, args, dev)
    wl = datagen.workload(args.workload)
    if wl.mode == "step":
        return bench_step(wl, args, dev)
    if args.which == "backward":
        return bench_backward(wl, args, dev)
    if args.which == "fused":
        return bench_fused(wl, args, dev)

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

    # measurement protocol, before the timed region: the device's achievable copy bandwidth
    # (the practical HBM ceiling) and cold calls (a 512 MB write before each, median of 20).
    # Together some tens of ms of GPU work, which also brings the GPU's clock up to its
    # steady state, whatever number of warmup steps is asked for.
    copy_gbs = copy_bandwidth(dev)
    cold_med, cold_min = _cold_median(step, stream, dev)

    # ---- timed region: W warmup steps, then exactly K steps back to back
    per_step, ev_avg = _time(step, args.steps, args.warmup, stream)

    if args.calib_copy:
        _calib_copy(dev)

    nbytes = algorithmic_bytes(wl, with_state=True)
    updates = wl.elements * wl.dstate
    hbm_gbs = nbytes / ev_avg / 1e9
    tflops = updates * FLOPS_PER_UPDATE / ev_avg / 1e12
    plan = sscan.forward_plan(wl.batch, wl.seqlen, wl.dim, wl.dstate, wl.io)
    lock = plan["kernel"] == "lockstep"
    # counter summaries: the lockstep kernel, or the segment path's kernels of one call together
    prof = f"k_lockstep_{wl.name}" if lock else f"k_seg_{wl.name}"
    sq = f"{prof}_sq_counters.md"
    kname = ("k_lockstep (timed: the whole sscan_forward call on its stream; the lockstep kernel is ~99% "
             "of it, the rest is the B/C staging launch)" if lock else
             f"k_seg + k_carry + k_segfix, {plan['segments']} segments of {plan['seg_len']} tokens: scan "
             f"from zero, carry of the segment end states, correction of the outputs (timed: the whole "
             f"sscan_forward call on its stream; traffic and VALU figures cover all kernels of one call)")
    roof = {
        "kernel": kname,
        "bound": "alu",
        "achieved": round(tflops, 3),
        "peak": PEAK_VALU_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tflops / PEAK_VALU_TFLOPS, 4),
        "traffic": recorded_traffic(f"{prof}_hbm_counters.md", FWD_SOURCES),
        "per_launch": {"updates": updates, "flops_per_update": FLOPS_PER_UPDATE,
                       "algorithmic_bytes": nbytes, "event_avg_us": round(ev_avg * 1e6, 2),
                       "cold_median_us": round(cold_med * 1e6, 2), "cold_min_us": round(cold_min * 1e6, 2),
                       "cold_runs": COLD_RUNS, "flush_bytes": FLUSH_BYTES},
        "hbm": {"achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / PEAK_HBM_GBS, 4),
                "cold_median_frac": round(nbytes / cold_med / 1e9 / PEAK_HBM_GBS, 4),
                "copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(hbm_gbs / copy_gbs, 4)},
        # from the committed SQ counter summary of this kernel (null once the sources change)
        "valu_issue": recorded_value(sq, "valu_issue", FWD_SOURCES),
        "valu_insts_per_wave_token": recorded_value(sq, "valu_insts_per_wave_token", FWD_SOURCES),
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
        "copy_gbs": round(copy_gbs, 1),
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(wl),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
