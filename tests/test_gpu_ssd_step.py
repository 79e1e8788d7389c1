"""GPU parity of sscan_ssd_step (one decode step of the scalar-A-per-head scan) through
the C ABI.

The steps are checked against the oracle's scalar-A-per-head scan over the same tokens
(the oracle's y at token t is the output of step t, its final state the state after the
last step): both N (64, 128), groups, both I/O dtypes, an initial state, A = 0 and A > 0
heads, no skip; a prefill with sscan_ssd_forward handed over to steps; and a state view
that is not 16-byte aligned.  Gates: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle.compare import TOL, rel_err
from tests.gpuutil import announce, to_dev, to_host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import selective_state_space_77_amd as sscan  # noqa: E402


def _wl(name, batch, L, H, G, N, io):
    return datagen.SsdWorkload(name, 40, batch, L, H, 64, G, N, io)


def _steps(wl, inp, state, D=True, t0=0):
    """Run tokens t0.. of inp as decode steps on `state`; returns y (batch, L - t0, H, P)."""
    io = wl.io
    A = torch.from_numpy(inp["A"]).cuda()
    Dt = torch.from_numpy(inp["D"]).cuda() if D else None
    ys = []
    for t in range(t0, wl.seqlen):
        ys.append(to_host(sscan.ssd_step(state, to_dev(np.ascontiguousarray(inp["x"][:, t]), io),
                                         to_dev(np.ascontiguousarray(inp["delta"][:, t]), io), A,
                                         to_dev(np.ascontiguousarray(inp["B"][:, t]), io),
                                         to_dev(np.ascontiguousarray(inp["C"][:, t]), io), Dt)))
    torch.cuda.synchronize()
    return np.stack(ys, axis=1)


@pytest.mark.parametrize("batch,L,H,G,N,io,h0,D", [
    (2, 20, 4, 2, 64, "f32", False, True),
    (2, 20, 4, 1, 128, "f32", True, True),
    (3, 16, 6, 3, 128, "bf16", True, True),
    (1, 12, 2, 2, 64, "bf16", False, False),
])
def test_ssd_steps_match_the_oracle(batch, L, H, G, N, io, h0, D):
    wl = _wl(f"ssdstep{N}{io}", batch, L, H, G, N, io)
    announce(f"ssd steps b={batch} L={L} H={H} G={G} N={N} io={io} h0={h0} D={D}")
    inp = datagen.ssd_inputs(wl)
    s0 = (np.random.default_rng(5).standard_normal((batch, H, 64, N)).astype(np.float32) if h0 else None)
    state = torch.from_numpy(s0).cuda() if h0 else torch.zeros(batch, H, 64, N, device="cuda")
    y = _steps(wl, inp, state, D)
    yr, hr = oracle.ssd_forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"] if D else None,
                                h0=s0)
    ey, eh = rel_err(y, yr), rel_err(state.cpu().numpy(), hr)
    announce(f"  err(y)={ey:.3e} err(h)={eh:.3e}")
    assert ey <= TOL[io] and eh <= TOL[io], (ey, eh)


def test_ssd_steps_with_zero_and_positive_A():
    wl = _wl("ssdstep_a", 2, 10, 4, 2, 64, "f32")
    inp = datagen.ssd_inputs(wl)
    inp["A"] = np.array([0.0, 0.3, -1e-7, -2.0], np.float32)  # A = 0: gain = delta; A > 0 grows
    announce("ssd steps with A = 0, A > 0 and a tiny A")
    state = torch.zeros(2, 4, 64, 64, device="cuda")
    y = _steps(wl, inp, state)
    yr, hr = oracle.ssd_forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"])
    assert rel_err(y, yr) <= TOL["f32"] and rel_err(state.cpu().numpy(), hr) <= TOL["f32"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_ssd_prefill_then_decode_handover(io):
    """sscan_ssd_forward over the first 130 tokens (not a chunk boundary), then steps from
    its final state: together equal the oracle over the whole sequence."""
    wl = _wl(f"ssdhand{io}", 2, 150, 4, 2, 128, io)
    inp = datagen.ssd_inputs(wl)
    P = 130
    announce(f"ssd prefill {P} tokens then {wl.seqlen - P} steps, io={io}")
    up = lambda k: to_dev(np.ascontiguousarray(inp[k][:, :P]), io)
    state = torch.empty(2, 4, 64, 128, device="cuda")
    yp = sscan.ssd_forward(up("x"), up("delta"), torch.from_numpy(inp["A"]).cuda(), up("B"), up("C"),
                           torch.from_numpy(inp["D"]).cuda(), final_state=state)
    ys = _steps(wl, inp, state, t0=P)
    yr, hr = oracle.ssd_forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"])
    y = np.concatenate([to_host(yp), ys], axis=1)
    ey, eh = rel_err(y, yr), rel_err(state.cpu().numpy(), hr)
    announce(f"  err(y)={ey:.3e} err(h)={eh:.3e}")
    assert ey <= TOL[io] and eh <= TOL[io], (ey, eh)


def test_ssd_step_misaligned_state():
    """A state view that is not 16-byte aligned takes element accesses and still updates
    every element (and nothing outside the view)."""
    wl = _wl("ssdstep_mis", 1, 6, 2, 1, 64, "f32")
    inp = datagen.ssd_inputs(wl)
    n = 2 * 64 * 64
    buf = torch.zeros(n + 2, device="cuda")
    state = buf[1:1 + n].view(1, 2, 64, 64)
    y = _steps(wl, inp, state)
    yr, hr = oracle.ssd_forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"])
    assert rel_err(y, yr) <= TOL["f32"] and rel_err(state.cpu().numpy(), hr) <= TOL["f32"]
    assert buf[0].item() == 0.0 and buf[-1].item() == 0.0
