"""MI355X (gfx950) selective scan (S6) -- Python binding of libsscan.so.

Argument marshalling only: every step of the scan runs in the library's HIP
kernels.  PyTorch supplies device memory and the stream.  There is no CPU or
PyTorch fallback: if libsscan.so is missing or fails to load, importing this
package raises.

    forward(x, delta, A, B, C, Dskip=None, y=None, final_state=None, stream=None,
            initial_state=None)
    forward_noalloc(...)   the same without any device allocation (static scratch)
    forward_fused(x, conv_weight, delta_raw, A, B, C, Dskip=None, conv_bias=None, delta_bias=None,
                  activation=None, conv_state=None, initial_state=None, y=None, final_state=None,
                  conv_state_out=None, stream=None)
    backward(x, delta, A, B, C, dy, Dskip=None, initial_state=None, dfinal_state=None, ...)
    step(state, x_t, delta_t, A, B_t, C_t, Dskip=None, y_t=None, stream=None)
    ssd_forward(x, delta, A, B, C, Dskip=None, initial_state=None, y=None, final_state=None,
                stream=None)
    ssd_step(state, x_t, delta_t, A, B_t, C_t, Dskip=None, y_t=None, stream=None)
    step_fused(state, conv_state, x_t, conv_weight, delta_raw_t, A, B_t, C_t, Dskip=None,
               conv_bias=None, delta_bias=None, activation=None, y_t=None, stream=None)

Shapes and layouts follow include/sscan.h: x, delta, y (batch, L, dim); B, C
(batch, L, N); A (dim, N) fp32; Dskip (dim,) fp32; states (batch, dim, N) fp32.
x, delta, B, C (and y) are all float32 or all bfloat16.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsscan.so")
# debug build of the same sources: every kernel fills its LDS with NaN before use
POISON_LIB_PATH = os.path.join(_HERE, "libsscan_poison.so")

F32, BF16 = 0, 1
MAX_DSTATE = 16
MAX_DCONV = 4
ACT = {None: 0, "none": 0, "silu": 1}

STATUS = {0: "SSCAN_OK", -1: "SSCAN_ERR_NULL", -2: "SSCAN_ERR_SHAPE", -3: "SSCAN_ERR_UNSUPPORTED",
          -4: "SSCAN_ERR_ALIAS", -5: "SSCAN_ERR_HIP"}


class SScanError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class PlanInfo(ctypes.Structure):
    """sscan_plan_info of include/sscan.h."""
    _fields_ = [("kernel", ctypes.c_int32), ("segments", ctypes.c_int32), ("seg_len", ctypes.c_int64),
                ("tiles", ctypes.c_int64), ("chunk_tokens", ctypes.c_int64),
                ("scratch_bytes", ctypes.c_int64)]


PLAN_KERNEL = {1: "lockstep", 2: "segment"}


def _load(path: str = None) -> ctypes.CDLL:
    """Load the library (or another build of it, such as the LDS-poison debug build) and
    declare its entry points."""
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(path)
    vp, fp, i64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64
    lib.sscan_forward.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i64, i64, i64, i64, ctypes.c_int, vp]
    lib.sscan_forward.restype = ctypes.c_int
    lib.sscan_forward_from_state.argtypes = [vp, vp, fp, vp, vp, fp, fp, vp, fp, i64, i64, i64, i64,
                                             ctypes.c_int, vp]
    lib.sscan_forward_from_state.restype = ctypes.c_int
    lib.sscan_forward_noalloc.argtypes = [vp, vp, fp, vp, vp, fp, fp, vp, fp, i64, i64, i64, i64,
                                          ctypes.c_int, vp]
    lib.sscan_forward_noalloc.restype = ctypes.c_int
    lib.sscan_backward.argtypes = [vp, vp, fp, vp, vp, fp, fp, vp, fp, vp, vp, fp, fp, fp, fp, fp,
                                   i64, i64, i64, i64, ctypes.c_int, vp]
    lib.sscan_backward.restype = ctypes.c_int
    ci = ctypes.c_int
    lib.sscan_forward_fused.argtypes = [vp, fp, fp, ci, ci, vp, vp, fp, fp, vp, vp, fp, fp, vp, fp, vp,
                                        i64, i64, i64, i64, ci, vp]
    lib.sscan_forward_fused.restype = ctypes.c_int
    lib.sscan_step_fused.argtypes = [fp, vp, vp, fp, fp, ci, ci, vp, fp, fp, vp, vp, fp, vp,
                                     i64, i64, i64, ci, vp]
    lib.sscan_step_fused.restype = ctypes.c_int
    lib.sscan_ssd_forward.argtypes = [vp, vp, fp, vp, vp, fp, fp, vp, fp, i64, i64, i64, i64, i64, i64,
                                      ci, vp]
    lib.sscan_ssd_forward.restype = ctypes.c_int
    lib.sscan_ssd_step.argtypes = [fp, vp, vp, fp, vp, vp, fp, vp, i64, i64, i64, i64, i64, ci, vp]
    lib.sscan_ssd_step.restype = ctypes.c_int
    lib.sscan_step.argtypes = [fp, vp, vp, fp, vp, vp, fp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.sscan_step.restype = ctypes.c_int
    lib.sscan_forward_plan.argtypes = [i64, i64, i64, i64, ci, ctypes.POINTER(PlanInfo)]
    lib.sscan_forward_plan.restype = ctypes.c_int
    lib.sscan_status_string.argtypes = [ctypes.c_int]
    lib.sscan_status_string.restype = ctypes.c_char_p
    lib.sscan_last_error.argtypes = []
    lib.sscan_last_error.restype = ctypes.c_char_p
    lib.sscan_version.argtypes = []
    lib.sscan_version.restype = ctypes.c_int
    return lib


lib = _load()


def _check(rc: int) -> None:
    if rc != 0:
        detail = lib.sscan_last_error().decode() or lib.sscan_status_string(rc).decode()
        raise SScanError(rc, detail)


def forward_plan(batch: int, seqlen: int, dim: int, dstate: int, io_dtype) -> dict:
    """How sscan_forward would split a problem of this shape (host only, no GPU work):
    kernel ("lockstep" or "segment"), segments, seg_len, tiles, chunk_tokens, scratch_bytes.
    io_dtype: torch.float32 / torch.bfloat16 or "f32" / "bf16"."""
    io = {torch.float32: F32, torch.bfloat16: BF16, "f32": F32, "bf16": BF16}[io_dtype]
    info = PlanInfo()
    _check(lib.sscan_forward_plan(batch, seqlen, dim, dstate, io, ctypes.byref(info)))
    out = {f: getattr(info, f) for f, _ in PlanInfo._fields_}
    out["kernel"] = PLAN_KERNEL[out["kernel"]]
    return out


def _io_code(*ts: torch.Tensor) -> int:
    dt = ts[0].dtype
    if any(t.dtype != dt for t in ts):
        raise TypeError("x, delta, B, C and y must share one dtype")
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported I/O dtype {dt}; use float32 or bfloat16")


def _dev(t: torch.Tensor | None, name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    return t.data_ptr()


def _shape(t: torch.Tensor | None, name: str, shape) -> None:
    """An output buffer given by the caller must have the output's shape: the kernels
    write every element of it."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")


def _one_device(*ts: torch.Tensor | None) -> None:
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")


def _stream(stream, device) -> int:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream if isinstance(s, torch.cuda.Stream) else int(s)


def _forward(entry, x, delta, A, B, C, Dskip, y, final_state, stream, initial_state):
    batch, L, dim = x.shape
    N = A.shape[1]
    if delta.shape != x.shape or tuple(A.shape) != (dim, N) or B.shape != (batch, L, N) or C.shape != B.shape:
        raise ValueError("inconsistent shapes")
    if y is None:
        y = torch.empty_like(x)
    _shape(y, "y", x.shape)
    io = _io_code(x, delta, B, C, y)
    _one_device(x, delta, A, B, C, Dskip, y, final_state, initial_state)
    if Dskip is not None and tuple(Dskip.shape) != (dim,):
        raise ValueError("Dskip must have shape (dim,)")
    if final_state is not None and tuple(final_state.shape) != (batch, dim, N):
        raise ValueError("final_state must have shape (batch, dim, N)")
    if initial_state is not None and tuple(initial_state.shape) != (batch, dim, N):
        raise ValueError("initial_state must have shape (batch, dim, N)")
    rc = entry(_dev(x, "x"), _dev(delta, "delta"), _dev(A, "A", torch.float32),
               _dev(B, "B"), _dev(C, "C"), _dev(Dskip, "Dskip", torch.float32),
               _dev(initial_state, "initial_state", torch.float32),
               _dev(y, "y"), _dev(final_state, "final_state", torch.float32),
               batch, L, dim, N, io, _stream(stream, x.device))
    _check(rc)
    return y


def forward(x, delta, A, B, C, Dskip=None, y=None, final_state=None, stream=None,
            initial_state=None):
    """Whole-sequence selective scan; returns y (written into `y` when given).

    initial_state: (batch, dim, N) fp32 state before the first token (default zero)."""
    return _forward(lib.sscan_forward_from_state, x, delta, A, B, C, Dskip, y, final_state, stream,
                    initial_state)


def forward_noalloc(x, delta, A, B, C, Dskip=None, y=None, final_state=None, stream=None,
                    initial_state=None):
    """forward() through sscan_forward_noalloc: no device allocation (the library's static
    per-GPU scratch, 64 MiB); pass y (and final_state) to allocate nothing at all.  Calls
    that overlap on one GPU race (they share that scratch)."""
    return _forward(lib.sscan_forward_noalloc, x, delta, A, B, C, Dskip, y, final_state, stream,
                    initial_state)


def _act_code(activation) -> int:
    if activation not in ACT:
        raise ValueError(f"activation must be None, 'none' or 'silu', not {activation!r}")
    return ACT[activation]


def forward_fused(x, conv_weight, delta_raw, A, B, C, Dskip=None, conv_bias=None, delta_bias=None,
                  activation=None, conv_state=None, initial_state=None, y=None, final_state=None,
                  conv_state_out=None, stream=None):
    """Selective scan with the front end fused: u = act(causal depthwise conv(x)),
    delta = softplus(delta_raw + delta_bias), then the scan on (u, delta); returns y.

    conv_weight: (dim, d_conv) fp32; conv_state / conv_state_out: (batch, d_conv-1, dim) in
    x's dtype (the raw inputs before token 0 / of the last d_conv-1 tokens)."""
    batch, L, dim = x.shape
    N = A.shape[1]
    if conv_weight.dim() != 2 or conv_weight.shape[0] != dim:
        raise ValueError("conv_weight must have shape (dim, d_conv)")
    K = conv_weight.shape[1]
    if delta_raw.shape != x.shape or tuple(A.shape) != (dim, N) or B.shape != (batch, L, N) \
            or C.shape != B.shape:
        raise ValueError("inconsistent shapes")
    for t, name, shape in ((Dskip, "Dskip", (dim,)), (conv_bias, "conv_bias", (dim,)),
                           (delta_bias, "delta_bias", (dim,)),
                           (conv_state, "conv_state", (batch, K - 1, dim)),
                           (conv_state_out, "conv_state_out", (batch, K - 1, dim)),
                           (initial_state, "initial_state", (batch, dim, N)),
                           (final_state, "final_state", (batch, dim, N))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
    if y is None:
        y = torch.empty_like(x)
    _shape(y, "y", x.shape)
    io = _io_code(x, delta_raw, B, C, y, *(t for t in (conv_state, conv_state_out) if t is not None))
    _one_device(x, conv_weight, delta_raw, A, B, C, Dskip, conv_bias, delta_bias, conv_state,
                initial_state, y, final_state, conv_state_out)
    rc = lib.sscan_forward_fused(
        _dev(x, "x"), _dev(conv_weight, "conv_weight", torch.float32),
        _dev(conv_bias, "conv_bias", torch.float32), K, _act_code(activation),
        _dev(conv_state, "conv_state"), _dev(delta_raw, "delta_raw"),
        _dev(delta_bias, "delta_bias", torch.float32), _dev(A, "A", torch.float32), _dev(B, "B"),
        _dev(C, "C"), _dev(Dskip, "Dskip", torch.float32),
        _dev(initial_state, "initial_state", torch.float32), _dev(y, "y"),
        _dev(final_state, "final_state", torch.float32), _dev(conv_state_out, "conv_state_out"),
        batch, L, dim, N, io, _stream(stream, x.device))
    _check(rc)
    return y


def step_fused(state, conv_state, x_t, conv_weight, delta_raw_t, A, B_t, C_t, Dskip=None,
               conv_bias=None, delta_bias=None, activation=None, y_t=None, stream=None):
    """One decode step with the front end fused; updates `state` and `conv_state`
    ((batch, d_conv-1, dim), x_t's dtype) in place and returns y_t."""
    batch, dim, N = state.shape
    K = conv_weight.shape[1]
    if x_t.shape != (batch, dim) or delta_raw_t.shape != (batch, dim) or tuple(A.shape) != (dim, N) \
            or B_t.shape != (batch, N) or C_t.shape != (batch, N) or tuple(conv_weight.shape) != (dim, K):
        raise ValueError("inconsistent shapes")
    if conv_state is not None and tuple(conv_state.shape) != (batch, K - 1, dim):
        raise ValueError("conv_state must have shape (batch, d_conv-1, dim)")
    if y_t is None:
        y_t = torch.empty_like(x_t)
    _shape(y_t, "y_t", x_t.shape)
    if Dskip is not None and tuple(Dskip.shape) != (dim,):
        raise ValueError("Dskip must have shape (dim,)")
    for t, name in ((conv_bias, "conv_bias"), (delta_bias, "delta_bias")):
        if t is not None and tuple(t.shape) != (dim,):
            raise ValueError(f"{name} must have shape (dim,)")
    io = _io_code(x_t, delta_raw_t, B_t, C_t, y_t, *(() if conv_state is None else (conv_state,)))
    _one_device(state, conv_state, x_t, conv_weight, delta_raw_t, A, B_t, C_t, Dskip, conv_bias,
                delta_bias, y_t)
    rc = lib.sscan_step_fused(
        _dev(state, "state", torch.float32), _dev(conv_state, "conv_state"), _dev(x_t, "x_t"),
        _dev(conv_weight, "conv_weight", torch.float32), _dev(conv_bias, "conv_bias", torch.float32),
        K, _act_code(activation), _dev(delta_raw_t, "delta_raw_t"),
        _dev(delta_bias, "delta_bias", torch.float32), _dev(A, "A", torch.float32), _dev(B_t, "B_t"),
        _dev(C_t, "C_t"), _dev(Dskip, "Dskip", torch.float32), _dev(y_t, "y_t"), batch, dim, N, io,
        _stream(stream, state.device))
    _check(rc)
    return y_t


def backward(x, delta, A, B, C, dy, Dskip=None, initial_state=None, dfinal_state=None,
             want_dskip=True, want_dinitial=True, stream=None):
    """Gradients of a scalar loss through forward(), given dy = dLoss/dy and
    dfinal_state = dLoss/d(final state) (None: zero).

    Returns a dict: dx, ddelta (like x), dA (dim, N), dB, dC (batch, L, N) fp32,
    dDskip (dim,) and dinitial_state (batch, dim, N) fp32 when wanted (else None)."""
    batch, L, dim = x.shape
    N = A.shape[1]
    if delta.shape != x.shape or dy.shape != x.shape or tuple(A.shape) != (dim, N) \
            or B.shape != (batch, L, N) or C.shape != B.shape:
        raise ValueError("inconsistent shapes")
    io = _io_code(x, delta, B, C, dy)
    _one_device(x, delta, A, B, C, dy, Dskip, initial_state, dfinal_state)
    for t, name, shape in ((Dskip, "Dskip", (dim,)), (initial_state, "initial_state", (batch, dim, N)),
                           (dfinal_state, "dfinal_state", (batch, dim, N))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
    f32 = dict(dtype=torch.float32, device=x.device)
    out = {"dx": torch.empty_like(x), "ddelta": torch.empty_like(x),
           "dA": torch.empty((dim, N), **f32), "dB": torch.empty((batch, L, N), **f32),
           "dC": torch.empty((batch, L, N), **f32),
           "dDskip": torch.empty((dim,), **f32) if want_dskip else None,
           "dinitial_state": torch.empty((batch, dim, N), **f32) if want_dinitial else None}
    rc = lib.sscan_backward(_dev(x, "x"), _dev(delta, "delta"), _dev(A, "A", torch.float32),
                            _dev(B, "B"), _dev(C, "C"), _dev(Dskip, "Dskip", torch.float32),
                            _dev(initial_state, "initial_state", torch.float32), _dev(dy, "dy"),
                            _dev(dfinal_state, "dfinal_state", torch.float32),
                            _dev(out["dx"], "dx"), _dev(out["ddelta"], "ddelta"), _dev(out["dA"], "dA"),
                            _dev(out["dB"], "dB"), _dev(out["dC"], "dC"), _dev(out["dDskip"], "dDskip"),
                            _dev(out["dinitial_state"], "dinitial_state"), batch, L, dim, N, io,
                            _stream(stream, x.device))
    _check(rc)
    return out


def step(state, x_t, delta_t, A, B_t, C_t, Dskip=None, y_t=None, stream=None):
    """One decode step; updates `state` in place and returns y_t."""
    batch, dim, N = state.shape
    if x_t.shape != (batch, dim) or delta_t.shape != (batch, dim) or tuple(A.shape) != (dim, N) \
            or B_t.shape != (batch, N) or C_t.shape != (batch, N):
        raise ValueError("inconsistent shapes")
    if y_t is None:
        y_t = torch.empty_like(x_t)
    _shape(y_t, "y_t", x_t.shape)
    io = _io_code(x_t, delta_t, B_t, C_t, y_t)
    _one_device(state, x_t, delta_t, A, B_t, C_t, Dskip, y_t)
    if Dskip is not None and tuple(Dskip.shape) != (dim,):
        raise ValueError("Dskip must have shape (dim,)")
    rc = lib.sscan_step(_dev(state, "state", torch.float32), _dev(x_t, "x_t"), _dev(delta_t, "delta_t"),
                        _dev(A, "A", torch.float32), _dev(B_t, "B_t"), _dev(C_t, "C_t"),
                        _dev(Dskip, "Dskip", torch.float32), _dev(y_t, "y_t"), batch, dim, N, io,
                        _stream(stream, state.device))
    _check(rc)
    return y_t


def version() -> int:
    return lib.sscan_version()


def ssd_forward(x, delta, A, B, C, Dskip=None, initial_state=None, y=None, final_state=None,
                stream=None):
    """Scalar-A-per-head scan (Mamba-2's SSM) in its chunked matrix form; returns y.

    x, y: (batch, L, H, P) with P = 64; delta: (batch, L, H); A: (H,) fp32; B, C:
    (batch, L, G, N) with N in {64, 128} and G | H; Dskip: (H,) fp32; states:
    (batch, H, P, N) fp32."""
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(delta.shape) != (batch, L, H) or tuple(A.shape) != (H,) or B.shape != (batch, L, G, N) \
            or C.shape != B.shape:
        raise ValueError("inconsistent shapes")
    for t, name, shape in ((Dskip, "Dskip", (H,)), (initial_state, "initial_state", (batch, H, P, N)),
                           (final_state, "final_state", (batch, H, P, N))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
    if y is None:
        y = torch.empty_like(x)
    _shape(y, "y", x.shape)
    io = _io_code(x, delta, B, C, y)
    _one_device(x, delta, A, B, C, Dskip, initial_state, y, final_state)
    rc = lib.sscan_ssd_forward(_dev(x, "x"), _dev(delta, "delta"), _dev(A, "A", torch.float32),
                               _dev(B, "B"), _dev(C, "C"), _dev(Dskip, "Dskip", torch.float32),
                               _dev(initial_state, "initial_state", torch.float32), _dev(y, "y"),
                               _dev(final_state, "final_state", torch.float32), batch, L, H, P, G, N, io,
                               _stream(stream, x.device))
    _check(rc)
    return y


def ssd_step(state, x_t, delta_t, A, B_t, C_t, Dskip=None, y_t=None, stream=None):
    """One decode step of the scalar-A-per-head scan; updates `state` in place and
    returns y_t.

    state: (batch, H, P, N) fp32 with P = 64, N in {64, 128}; x_t, y_t: (batch, H, P);
    delta_t: (batch, H); A, Dskip: (H,) fp32; B_t, C_t: (batch, G, N) with G | H."""
    batch, H, P, N = state.shape
    G = B_t.shape[1] if B_t.dim() == 3 else -1
    if tuple(x_t.shape) != (batch, H, P) or tuple(delta_t.shape) != (batch, H) or tuple(A.shape) != (H,) \
            or tuple(B_t.shape) != (batch, G, N) or C_t.shape != B_t.shape:
        raise ValueError("inconsistent shapes")
    if Dskip is not None and tuple(Dskip.shape) != (H,):
        raise ValueError("Dskip must have shape (H,)")
    if y_t is None:
        y_t = torch.empty_like(x_t)
    _shape(y_t, "y_t", x_t.shape)
    io = _io_code(x_t, delta_t, B_t, C_t, y_t)
    _one_device(state, x_t, delta_t, A, B_t, C_t, Dskip, y_t)
    rc = lib.sscan_ssd_step(_dev(state, "state", torch.float32), _dev(x_t, "x_t"), _dev(delta_t, "delta_t"),
                            _dev(A, "A", torch.float32), _dev(B_t, "B_t"), _dev(C_t, "C_t"),
                            _dev(Dskip, "Dskip", torch.float32), _dev(y_t, "y_t"), batch, H, P, G, N, io,
                            _stream(stream, state.device))
    _check(rc)
    return y_t
