"""Seeded synthetic inputs for the selective-scan (S6) workloads.

This module is the single source of inputs for both the HIP path and the fp64
oracle.  It holds none of the scan's arithmetic (no discretisation, no
recurrence, no readout): only random draws, the input distributions, and the
fp32 -> bf16 round-to-nearest-even encoding of the draws.

Distributions (the recipe each workload below states):
  x, B, C      ~ N(0, 1), drawn per element.
  Dskip[d]     ~ N(0, 1), one value per channel, fp32.
  A[d, n]      "loguniform":  -exp(U(log 0.5, log 4)) per (d, n)
               "s4d_real":    -(n + 1) for every channel d.
  delta        softplus(0.5 * N(0, 1) + bias[d]) with a per-channel bias
               bias[d] = log(expm1(U(1e-3, 1e-1))), i.e. the inverse softplus
               of a step drawn uniformly from [1e-3, 1e-1].
               (Mamba feeds softplus(Linear(x_t) + bias); the bias is what
               sets the step range, "Mamba and State Space Models",
               pseudocode under "Mamba: making the state selective" and the
               dt_min/dt_max dial under "How this shows up in practice".)

Every draw is made in fp64, rounded to fp32 and then, for bf16 workloads,
rounded to bf16 (RNE).  Values are returned as float32 arrays that hold
exactly the values the device sees; `bf16_bits` gives the raw 16-bit
patterns for upload.

Streams.  Each tensor has its own numpy PCG64 stream keyed by
(seed, workload key, tensor id, batch row, block index).  Sequence tensors
are drawn in blocks of TBLK tokens, so any token range can be regenerated
without drawing the rest of the sequence (needed for the 2^20-token
workload).  Decode-step workloads key their streams by step index instead.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

TBLK = 256  # tokens per generator block

_TENSOR_IDS = {"x": 1, "delta": 2, "B": 3, "C": 4, "A": 5, "Dskip": 6, "dt_bias": 7,
               "dy": 8, "h0": 9, "dhT": 10, "delta_raw": 11, "conv_w": 12, "conv_b": 13,
               "conv_state": 14}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, I/O dtype and how A is initialised."""

    name: str
    key: int  # stream key, fixed per workload
    batch: int
    seqlen: int  # tokens per sequence (decode workloads: number of steps)
    dim: int  # channels
    dstate: int  # N, states per channel
    io: str  # "f32" or "bf16": dtype of x, delta, B, C and y
    a_init: str  # "loguniform" or "s4d_real"
    mode: str = "scan"  # "scan" (whole sequence) or "step" (one token per call)

    @property
    def elements(self) -> int:
        """B*L*D: channel-token elements the workload covers."""
        return self.batch * self.seqlen * self.dim


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", 0, 1, 256, 16, 4, "f32", "loguniform"),
        Workload("mamba130m_f32", 1, 8, 2048, 1536, 16, "f32", "s4d_real"),
        Workload("mamba1p4b_bf16", 2, 4, 8192, 4096, 16, "bf16", "s4d_real"),
        Workload("long1m_bf16", 3, 1, 1 << 20, 2048, 16, "bf16", "s4d_real"),
        Workload("decode_bf16", 4, 256, 1000, 5120, 16, "bf16", "s4d_real", mode="step"),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def custom(name: str, batch: int, seqlen: int, dim: int, dstate: int, io: str = "f32",
           a_init: str = "loguniform", key: int = 100, mode: str = "scan") -> Workload:
    """An ad-hoc workload (edge shapes in tests), same distributions."""
    return Workload(name, key, batch, seqlen, dim, dstate, io, a_init, mode)


# ----------------------------------------------------------------------------- encoding

def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); result is float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # uint32 cannot overflow here for non-NaN inputs (largest: 0xFF7FFFFF + 0x8000)
    nan = np.isnan(a)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    r &= np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """16-bit patterns of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable; call round_bf16 first")
    return (u >> 16).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """float32 values of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _to_io(v64: np.ndarray, io: str) -> np.ndarray:
    v = v64.astype(np.float32)
    return round_bf16(v) if io == "bf16" else v


# ----------------------------------------------------------------------------- streams

def _rng(seed: int, wl: Workload, tensor: str, *idx: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, wl.key, _TENSOR_IDS[tensor], *idx])))


def gen_A(wl: Workload, seed: int = 0) -> np.ndarray:
    """A[d, n] (fp32, shape (dim, N))."""
    if wl.a_init == "s4d_real":
        row = -np.arange(1, wl.dstate + 1, dtype=np.float64)
        return np.ascontiguousarray(np.broadcast_to(row, (wl.dim, wl.dstate)), dtype=np.float32)
    if wl.a_init == "loguniform":
        u = _rng(seed, wl, "A").uniform(np.log(0.5), np.log(4.0), size=(wl.dim, wl.dstate))
        return (-np.exp(u)).astype(np.float32)
    raise ValueError(f"unknown a_init {wl.a_init!r}")


def gen_Dskip(wl: Workload, seed: int = 0) -> np.ndarray:
    """Dskip[d] (fp32, shape (dim,))."""
    return _rng(seed, wl, "Dskip").standard_normal(wl.dim).astype(np.float32)


def gen_dt_bias(wl: Workload, seed: int = 0) -> np.ndarray:
    """Per-channel softplus bias of the step size (fp64, shape (dim,))."""
    u = _rng(seed, wl, "dt_bias").uniform(1e-3, 1e-1, size=wl.dim)
    return np.log(np.expm1(u))


def _width(wl: Workload, tensor: str) -> int:
    return wl.dim if tensor in ("x", "delta", "dy", "delta_raw") else wl.dstate


def _draw(g: np.random.Generator, shape, tensor: str, bias) -> np.ndarray:
    z = g.standard_normal(shape)
    if tensor == "delta":
        return np.logaddexp(0.0, 0.5 * z + bias)  # softplus of the biased draw
    if tensor == "delta_raw":
        return 0.5 * z                             # the same draw before bias and softplus
    return z


def gen_block(wl: Workload, tensor: str, b: int, blk: int, seed: int = 0,
              bias: np.ndarray | None = None) -> np.ndarray:
    """Tokens [blk*TBLK, min((blk+1)*TBLK, L)) of batch row b: (rows, width) float32."""
    t0 = blk * TBLK
    rows = min(TBLK, wl.seqlen - t0)
    if rows <= 0:
        raise IndexError("block past the end of the sequence")
    if tensor == "delta" and bias is None:
        bias = gen_dt_bias(wl, seed)
    v = _draw(_rng(seed, wl, tensor, b, blk), (rows, _width(wl, tensor)), tensor, bias)
    return _to_io(v, wl.io)


def _threads(threads: int | None) -> int:
    if threads is not None:
        return max(1, threads)
    return max(1, min(16, os.cpu_count() or 1))


def gen_seq(wl: Workload, tensor: str, t0: int = 0, t1: int | None = None, seed: int = 0,
            batch_rows=None, threads: int | None = None) -> np.ndarray:
    """Sequence tensor over tokens [t0, t1): float32 (batch, t1-t0, width)."""
    if wl.mode != "scan":
        raise ValueError("gen_seq is for whole-sequence workloads; use gen_step")
    t1 = wl.seqlen if t1 is None else t1
    rows_b = list(range(wl.batch)) if batch_rows is None else list(batch_rows)
    width = _width(wl, tensor)
    out = np.empty((len(rows_b), t1 - t0, width), dtype=np.float32)
    bias = gen_dt_bias(wl, seed) if tensor == "delta" else None
    jobs = [(i, b, blk) for i, b in enumerate(rows_b)
            for blk in range(t0 // TBLK, (t1 + TBLK - 1) // TBLK)]

    def one(job):
        i, b, blk = job
        v = gen_block(wl, tensor, b, blk, seed, bias)
        s = blk * TBLK
        lo, hi = max(t0, s), min(t1, s + v.shape[0])
        out[i, lo - t0:hi - t0] = v[lo - s:hi - s]

    if len(jobs) == 1:
        one(jobs[0])
    else:
        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(one, jobs))
    return out


def gen_step(wl: Workload, tensor: str, step: int, seed: int = 0,
             bias: np.ndarray | None = None) -> np.ndarray:
    """Decode-step tensor for one step: float32 (batch, width)."""
    if wl.mode != "step":
        raise ValueError("gen_step is for decode-step workloads")
    if tensor == "delta" and bias is None:
        bias = gen_dt_bias(wl, seed)
    v = _draw(_rng(seed, wl, tensor, step), (wl.batch, _width(wl, tensor)), tensor, bias)
    return _to_io(v, wl.io)


def scan_inputs(wl: Workload, seed: int = 0, t0: int = 0, t1: int | None = None,
                threads: int | None = None) -> dict:
    """All inputs of a whole-sequence workload over tokens [t0, t1) (float32 arrays)."""
    return {
        "x": gen_seq(wl, "x", t0, t1, seed, threads=threads),
        "delta": gen_seq(wl, "delta", t0, t1, seed, threads=threads),
        "A": gen_A(wl, seed),
        "B": gen_seq(wl, "B", t0, t1, seed, threads=threads),
        "C": gen_seq(wl, "C", t0, t1, seed, threads=threads),
        "Dskip": gen_Dskip(wl, seed),
    }


def step_inputs(wl: Workload, step: int, seed: int = 0, bias: np.ndarray | None = None) -> dict:
    """Per-step inputs of a decode workload (A and Dskip are per workload)."""
    if bias is None:
        bias = gen_dt_bias(wl, seed)
    return {t: gen_step(wl, t, step, seed, bias) for t in ("x", "delta", "B", "C")}


def gen_state(wl: Workload, tensor: str, seed: int = 0) -> np.ndarray:
    """A (batch, dim, N) fp32 state-shaped tensor, standard normal: "h0" (state
    before token 0) or "dhT" (cotangent of the final state)."""
    if tensor not in ("h0", "dhT"):
        raise ValueError(f"not a state tensor: {tensor!r}")
    g = _rng(seed, wl, tensor)
    return g.standard_normal((wl.batch, wl.dim, wl.dstate)).astype(np.float32)


def grad_inputs(wl: Workload, seed: int = 0, threads: int | None = None) -> dict:
    """Cotangents for a backward pass: dy (batch, L, dim) in the I/O dtype's values,
    standard normal like x, and dhT; plus an initial state h0."""
    return {"dy": gen_seq(wl, "dy", seed=seed, threads=threads),
            "h0": gen_state(wl, "h0", seed), "dhT": gen_state(wl, "dhT", seed)}


def frontend_inputs(wl: Workload, d_conv: int, seed: int = 0, threads: int | None = None) -> dict:
    """Inputs of the fused front end: delta_raw (batch, L, dim) = 0.5 N(0,1) in the I/O
    dtype's values (with delta_bias below, softplus(delta_raw + delta_bias) has the
    distribution of the generated delta), delta_bias = the per-channel dt bias (fp32),
    conv_w (dim, d_conv) and conv_b (dim) ~ U(-1/sqrt(d_conv), 1/sqrt(d_conv)) fp32, and
    conv_state (batch, d_conv-1, dim) ~ N(0,1) in the I/O dtype's values.  The raw
    convolution input is gen_seq(wl, "x")."""
    lim = 1.0 / np.sqrt(d_conv)
    return {
        "delta_raw": gen_seq(wl, "delta_raw", seed=seed, threads=threads),
        "delta_bias": gen_dt_bias(wl, seed).astype(np.float32),
        "conv_w": _rng(seed, wl, "conv_w").uniform(-lim, lim, (wl.dim, d_conv)).astype(np.float32),
        "conv_b": _rng(seed, wl, "conv_b").uniform(-lim, lim, wl.dim).astype(np.float32),
        "conv_state": _to_io(_rng(seed, wl, "conv_state").standard_normal((wl.batch, d_conv - 1, wl.dim)),
                             wl.io),
    }


# ----------------------------------------------------------------------------- scalar A per head

@dataclass(frozen=True)
class SsdWorkload:
    """A Mamba-2-shaped workload: heads of P channels, scalar A per head, B/C per group."""
    name: str
    key: int
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    io: str
    mode: str = "scan"  # "step": seqlen tokens staged for decode steps

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.nheads * self.headdim


SSD_WORKLOADS = {
    w.name: w for w in (
        # inner width 4096 (64 heads x 64) as the benchmarked per-channel workload, N = 128
        SsdWorkload("mamba2_bf16", 20, 4, 8192, 64, 64, 1, 128, "bf16"),
        SsdWorkload("mamba2_small_f32", 21, 2, 1000, 8, 64, 2, 64, "f32"),
        # decode steps at the same width: 64 sequences, 128 MB fp32 state, 64 staged tokens
        SsdWorkload("mamba2_decode_bf16", 22, 64, 64, 64, 64, 1, 128, "bf16", mode="step"),
    )
}


def ssd_inputs(wl: SsdWorkload, seed: int = 0) -> dict:
    """x (batch, L, H, P), B, C (batch, L, G, N) ~ N(0,1); delta (batch, L, H) =
    softplus(0.5 N(0,1) + per-head dt bias); A (H) = -exp(U(log 1, log 16)); D (H) ~ N(0,1).
    Sequence tensors in the I/O dtype's values; A, D fp32."""
    def rng(tensor):
        return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
            [seed, wl.key, _TENSOR_IDS[tensor], 1000])))
    b, L, H, P, G, N = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.ngroups, wl.dstate
    bias = np.log(np.expm1(rng("dt_bias").uniform(1e-3, 1e-1, H)))
    return {
        "x": _to_io(rng("x").standard_normal((b, L, H, P)), wl.io),
        "delta": _to_io(np.logaddexp(0.0, 0.5 * rng("delta").standard_normal((b, L, H)) + bias), wl.io),
        "A": (-np.exp(rng("A").uniform(0.0, np.log(16.0), H))).astype(np.float32),
        "B": _to_io(rng("B").standard_normal((b, L, G, N)), wl.io),
        "C": _to_io(rng("C").standard_normal((b, L, G, N)), wl.io),
        "D": rng("Dskip").standard_normal(H).astype(np.float32),
    }
