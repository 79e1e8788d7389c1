"""fp64 CPU oracle of the selective scan (S6) -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of
bench.py may import this package.  The product path (the HIP library and its
Python binding) never imports or calls it, and the two share no code.

The arithmetic lives in sscan_oracle.c (plain C, fp64, libm exp/expm1); this
module only builds/loads it and marshals numpy arrays.  Inputs are upcast to
fp64 from exactly the values the device sees (bf16-rounded where the workload
is bf16); outputs stay fp64.  See sscan_oracle.c for the definition and the
passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sscan_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, no fast-math: libm exp/expm1 as written)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                        "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_forward.argtypes = [dp] * 9 + [i64] * 4 + [ctypes.c_int]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_step.argtypes = [dp] * 8 + [i64] * 3
        lib.oracle_step.restype = ctypes.c_int
        lib.oracle_backward.argtypes = [dp] * 16 + [i64] * 4 + [ctypes.c_int]
        lib.oracle_backward.restype = ctypes.c_int
        lib.oracle_frontend.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, dp,
                                        i64, i64, i64]
        lib.oracle_frontend.restype = ctypes.c_int
        lib.oracle_ssd_forward.argtypes = [dp] * 9 + [i64] * 6 + [ctypes.c_int]
        lib.oracle_ssd_forward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def forward(x, delta, A, B, C, Dskip=None, h0=None, nthreads: int = 1, want_state: bool = True):
    """Sequential fp64 forward pass.

    x, delta: (batch, L, dim); A: (dim, N); B, C: (batch, L, N); Dskip: (dim,) or None;
    h0: (batch, dim, N) or None (zero start).  Returns (y, final_state) in fp64;
    final_state is None when want_state is False.
    """
    x, delta, A, B, C = map(_f64, (x, delta, A, B, C))
    Dskip, h0 = _f64(Dskip), _f64(h0)
    batch, L, dim = x.shape
    N = A.shape[1]
    if delta.shape != x.shape or A.shape != (dim, N) or B.shape != (batch, L, N) or C.shape != B.shape:
        raise ValueError("inconsistent shapes")
    if Dskip is not None and Dskip.shape != (dim,):
        raise ValueError("Dskip must have shape (dim,)")
    if h0 is not None and h0.shape != (batch, dim, N):
        raise ValueError("h0 must have shape (batch, dim, N)")
    y = np.empty((batch, L, dim), dtype=np.float64)
    hs = np.empty((batch, dim, N), dtype=np.float64) if want_state else None
    rc = _load().oracle_forward(_p(x), _p(delta), _p(A), _p(B), _p(C), _p(Dskip), _p(h0),
                                _p(y), _p(hs), batch, L, dim, N, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_forward failed ({rc})")
    return y, hs


def step(state, x_t, delta_t, A, B_t, C_t, Dskip=None):
    """One fp64 decode step; returns (y_t, new_state) and leaves `state` untouched.

    state: (batch, dim, N); x_t, delta_t: (batch, dim); B_t, C_t: (batch, N).
    """
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    x_t, delta_t, A, B_t, C_t, Dskip = map(_f64, (x_t, delta_t, A, B_t, C_t, Dskip))
    batch, dim, N = st.shape
    if x_t.shape != (batch, dim) or delta_t.shape != (batch, dim) or A.shape != (dim, N) \
            or B_t.shape != (batch, N) or C_t.shape != (batch, N):
        raise ValueError("inconsistent shapes")
    y = np.empty((batch, dim), dtype=np.float64)
    rc = _load().oracle_step(_p(st), _p(x_t), _p(delta_t), _p(A), _p(B_t), _p(C_t), _p(Dskip),
                             _p(y), batch, dim, N)
    if rc != 0:
        raise RuntimeError(f"oracle_step failed ({rc})")
    return y, st


def backward(x, delta, A, B, C, Dskip, dy, h0=None, dhT=None, nthreads: int = 1):
    """fp64 gradients of sum(dy * y) + sum(dhT * final_state) through forward().

    Returns a dict with dx, ddelta (batch, L, dim), dA (dim, N), dB, dC (batch, L, N),
    dDskip (dim,) and dh0 (batch, dim, N).  Dskip None means a zero skip (dDskip is
    still returned)."""
    x, delta, A, B, C, dy = map(_f64, (x, delta, A, B, C, dy))
    Dskip, h0, dhT = _f64(Dskip), _f64(h0), _f64(dhT)
    batch, L, dim = x.shape
    N = A.shape[1]
    if dy.shape != x.shape or delta.shape != x.shape or B.shape != (batch, L, N) or C.shape != B.shape:
        raise ValueError("inconsistent shapes")
    out = {"dx": np.empty_like(x), "ddelta": np.empty_like(x), "dA": np.empty((dim, N)),
           "dB": np.empty((batch, L, N)), "dC": np.empty((batch, L, N)), "dDskip": np.empty(dim),
           "dh0": np.empty((batch, dim, N))}
    rc = _load().oracle_backward(_p(x), _p(delta), _p(A), _p(B), _p(C), _p(Dskip), _p(h0), _p(dy),
                                 _p(dhT), _p(out["dx"]), _p(out["ddelta"]), _p(out["dA"]),
                                 _p(out["dB"]), _p(out["dC"]), _p(out["dDskip"]), _p(out["dh0"]),
                                 batch, L, dim, N, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_backward failed ({rc})")
    return out


def frontend(xin, conv_w, delta_raw, conv_bias=None, delta_bias=None, act: int = 0,
             conv_state=None):
    """fp64 front end: (u, delta, conv_state_out).

    xin, delta_raw: (batch, L, dim); conv_w: (dim, K); conv_bias, delta_bias: (dim,) or None;
    act: 0 none, 1 SiLU; conv_state: (batch, K-1, dim) inputs before token 0, or None (zeros).
    u = act(causal depthwise convolution of xin), delta = softplus(delta_raw + delta_bias),
    conv_state_out = the last K-1 inputs, (batch, K-1, dim)."""
    xin, conv_w, delta_raw = map(_f64, (xin, conv_w, delta_raw))
    conv_bias, delta_bias, conv_state = map(_f64, (conv_bias, delta_bias, conv_state))
    batch, L, dim = xin.shape
    K = conv_w.shape[1]
    if delta_raw.shape != xin.shape or conv_w.shape != (dim, K):
        raise ValueError("inconsistent shapes")
    if conv_state is not None and conv_state.shape != (batch, K - 1, dim):
        raise ValueError("conv_state must have shape (batch, K-1, dim)")
    u = np.empty_like(xin)
    delta = np.empty_like(xin)
    cs = np.empty((batch, K - 1, dim))
    rc = _load().oracle_frontend(_p(xin), _p(conv_w), _p(conv_bias), K, int(act), _p(conv_state),
                                 _p(delta_raw), _p(delta_bias), _p(u), _p(delta), _p(cs), batch, L, dim)
    if rc != 0:
        raise RuntimeError(f"oracle_frontend failed ({rc})")
    return u, delta, cs


def forward_fused(xin, conv_w, delta_raw, A, B, C, Dskip=None, conv_bias=None, delta_bias=None,
                  act: int = 0, conv_state=None, h0=None, nthreads: int = 1):
    """The fused entry point's definition: frontend() then forward() on its outputs.
    Returns (y, final_state, conv_state_out)."""
    u, delta, cs = frontend(xin, conv_w, delta_raw, conv_bias, delta_bias, act, conv_state)
    y, hs = forward(u, delta, A, B, C, Dskip, h0=h0, nthreads=nthreads)
    return y, hs, cs


def ssd_forward(x, delta, A, B, C, D=None, h0=None, want_state: bool = True, nthreads: int = 1):
    """fp64 scalar-A-per-head scan (Mamba-2's SSM); rows (b, h, p) split over nthreads.

    x: (batch, L, H, P); delta: (batch, L, H); A: (H,); B, C: (batch, L, G, N) with G | H;
    D: (H,) or None; h0: (batch, H, P, N) or None.  Returns (y (batch, L, H, P), final state
    (batch, H, P, N) or None)."""
    x, delta, A, B, C = map(_f64, (x, delta, A, B, C))
    D, h0 = _f64(D), _f64(h0)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if delta.shape != (batch, L, H) or A.shape != (H,) or B.shape != (batch, L, G, N) \
            or C.shape != B.shape or H % G:
        raise ValueError("inconsistent shapes")
    if D is not None and D.shape != (H,):
        raise ValueError("D must have shape (H,)")
    if h0 is not None and h0.shape != (batch, H, P, N):
        raise ValueError("h0 must have shape (batch, H, P, N)")
    y = np.empty_like(x)
    hT = np.empty((batch, H, P, N)) if want_state else None
    rc = _load().oracle_ssd_forward(_p(x), _p(delta), _p(A), _p(B), _p(C), _p(D), _p(h0), _p(y), _p(hT),
                                    batch, L, H, P, G, N, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_ssd_forward failed ({rc})")
    return y, hT
