"""GPU parity of sscan_ssd_forward (scalar A per head, chunked matrix form on MFMA) against
the fp64 oracle's scalar-A-per-head scan, through the C ABI.

Small shapes are compared on every output and the final state: both N (64, 128), groups,
ragged L around the 64-token chunk, L = 1, an initial state, A = 0 and A > 0 heads,
no skip.  The 4 x 8192 x (64 heads x 64) bf16, N = 128 workload runs whole on the GPU and
is compared on every output and the whole final state (the oracle splits its independent
(batch row, head, channel) rows over threads).  Gates: 1e-4 for fp32 inputs (fp32 matrix products), 2e-2 for bf16 inputs
(bf16 operands, fp32 accumulation and state).
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle.compare import TOL, rel_err
from tests.gpuutil import announce, oracle_threads, to_dev, to_host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import selective_state_space_77_amd as sscan  # noqa: E402


def _up(inp, io):
    t = {k: to_dev(inp[k], io) for k in ("x", "delta", "B", "C")}
    t["A"] = torch.from_numpy(inp["A"]).cuda()
    t["D"] = torch.from_numpy(inp["D"]).cuda()
    return t


def _run(wl, inp, h0=None, D=True):
    t = _up(inp, wl.io)
    hs = torch.full((wl.batch, wl.nheads, wl.headdim, wl.dstate), float("nan"), device="cuda")
    y = sscan.ssd_forward(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"] if D else None,
                          initial_state=None if h0 is None else torch.from_numpy(h0).cuda(), final_state=hs)
    torch.cuda.synchronize()
    return to_host(y), hs.cpu().numpy()


def _check(wl, inp=None, h0=None, D=True):
    announce(f"ssd {wl.name} b={wl.batch} L={wl.seqlen} H={wl.nheads} P={wl.headdim} G={wl.ngroups} "
             f"N={wl.dstate} io={wl.io} h0={h0 is not None} D={D}")
    inp = inp or datagen.ssd_inputs(wl)
    y, hs = _run(wl, inp, h0, D)
    yr, hr = oracle.ssd_forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"] if D else None,
                                h0=h0)
    ey, eh = rel_err(y, yr), rel_err(hs, hr)
    announce(f"  err(y)={ey:.3e} err(h)={eh:.3e}")
    assert ey <= TOL[wl.io], ey
    assert eh <= TOL[wl.io], eh


def _wl(name, batch, L, H, G, N, io):
    return datagen.SsdWorkload(name, 30, batch, L, H, 64, G, N, io)


@pytest.mark.parametrize("batch,L,H,G,N,io", [
    (2, 1000, 8, 2, 64, "f32"),
    (2, 1000, 8, 2, 64, "bf16"),
    (1, 300, 4, 1, 128, "f32"),
    (2, 300, 4, 4, 128, "bf16"),
    (1, 64, 2, 1, 64, "f32"),       # exactly one chunk
    (1, 65, 2, 2, 128, "f32"),      # one token into the second chunk
    (3, 1, 2, 1, 64, "bf16"),       # one token
    (1, 37, 6, 3, 64, "f32"),       # one partial chunk, 3 groups
])
def test_ssd_shapes(batch, L, H, G, N, io):
    _check(_wl("ssd", batch, L, H, G, N, io))


def test_ssd_named_small_workload_with_initial_state():
    wl = datagen.SSD_WORKLOADS["mamba2_small_f32"]
    h0 = np.random.default_rng(7).standard_normal((wl.batch, wl.nheads, wl.headdim, wl.dstate)).astype(np.float32)
    _check(wl, h0=h0)
    _check(wl, D=False)


def test_ssd_zero_and_positive_A_heads():
    wl = _wl("ssd_A", 1, 400, 4, 1, 64, "f32")
    inp = datagen.ssd_inputs(wl)
    inp["A"] = np.array([0.0, 0.02, -1e-4, -30.0], np.float32)   # hold, slow growth, tiny, fast decay
    _check(wl, inp=inp)


def test_ssd_full_workload_every_head():
    wl = datagen.SSD_WORKLOADS["mamba2_bf16"]
    announce(f"ssd {wl.name}: full run, every head vs the oracle")
    inp = datagen.ssd_inputs(wl)
    y, hs = _run(wl, inp)
    yr, hr = oracle.ssd_forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                                nthreads=oracle_threads())
    ey, eh = rel_err(y, yr), rel_err(hs, hr)
    announce(f"  err(y)={ey:.3e} err(h)={eh:.3e}")
    assert np.isfinite(y).all()
    assert ey <= TOL[wl.io] and eh <= TOL[wl.io], (ey, eh)


def test_ssd_resumes_from_its_final_state():
    wl = _wl("ssd_resume", 2, 500, 4, 2, 128, "f32")
    inp = datagen.ssd_inputs(wl)
    announce("ssd split at 200 (not a chunk boundary) vs one pass")
    y, hs = _run(wl, inp)
    cut = 200
    part = lambda a, b: {k: (v[:, a:b] if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
    w1 = _wl("ssd_resume", 2, cut, 4, 2, 128, "f32")
    w2 = _wl("ssd_resume", 2, 500 - cut, 4, 2, 128, "f32")
    y1, h1 = _run(w1, part(0, cut))
    y2, h2 = _run(w2, part(cut, 500), h0=h1)
    e = rel_err(np.concatenate([y1, y2], axis=1), y.astype(np.float64))
    announce(f"  pieces vs one pass: {e:.3e}")
    assert e <= 1e-5 and rel_err(h2, hs.astype(np.float64)) <= 1e-5


def test_ssd_unaligned_bf16_inputs_take_the_elementwise_kernel():
    """x, B and C that are not 16-byte aligned (views one element in) give the same
    result through the element-by-element kernel."""
    wl = _wl("ssd_unal", 1, 200, 2, 1, 64, "bf16")
    inp = datagen.ssd_inputs(wl)
    announce("ssd unaligned bf16 inputs")
    y_ref, h_ref = _run(wl, inp)
    t = _up(inp, "bf16")
    def shifted(z):
        buf = torch.empty(z.numel() + 1, dtype=z.dtype, device="cuda")
        v = buf[1:].view(z.shape)
        v.copy_(z)
        return v
    x, B, C = shifted(t["x"]), shifted(t["B"]), shifted(t["C"])
    assert x.data_ptr() % 16 != 0
    hs = torch.empty(1, 2, 64, 64, device="cuda")
    y = sscan.ssd_forward(x, t["delta"], t["A"], B, C, t["D"], final_state=hs)
    torch.cuda.synchronize()
    yr, hr = oracle.ssd_forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"])
    assert rel_err(to_host(y), yr) <= TOL["bf16"] and rel_err(hs.cpu().numpy(), hr) <= TOL["bf16"]
    assert rel_err(to_host(y), y_ref.astype(np.float64)) <= 1e-2


def test_ssd_deterministic():
    wl = _wl("ssd_det", 2, 300, 4, 1, 128, "bf16")
    inp = datagen.ssd_inputs(wl)
    announce("ssd determinism")
    a, b = _run(wl, inp), _run(wl, inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
