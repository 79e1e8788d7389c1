"""GPU parity on seeded random shapes: the forward, backward, scalar-A-per-head and
decode-step entry points against the fp64 oracle, element by element.

Each case draws its shape and options from a fixed seed (so a failure names a
reproducible case): batch, sequence length (including 1 and lengths around the
kernels' run and chunk sizes), channel count (ragged against the 64-channel tile),
state size, I/O dtype, A kind (structured-real or log-uniform), and whether the skip,
an initial state or the final-state cotangent are passed.  Sizes stay small enough
for the oracle to finish in well under a second per case.  Gates as elsewhere: 1e-4
for fp32 inputs, 2e-2 for bf16 inputs (oracle.compare).
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle.compare import TOL, rel_err
from tests.gpuutil import announce, oracle_threads, to_dev, to_host, upload_scan

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import selective_state_space_77_amd as sscan  # noqa: E402


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    L = int(rng.choice([1, 2, 15, 16, 17, 31, 33, 64, 255, 257, int(rng.integers(3, 700))]))
    return dict(batch=int(rng.integers(1, 4)), L=L, dim=int(rng.integers(1, 300)),
                N=int(rng.integers(1, 17)), io=str(rng.choice(["f32", "bf16"])),
                a_init=str(rng.choice(["s4d_real", "loguniform"])), skip=bool(rng.integers(0, 2)),
                h0=bool(rng.integers(0, 2)), dhT=bool(rng.integers(0, 2)))


def _case(seed, mode="scan"):
    c = _draw(seed)
    wl = datagen.custom(f"rand{seed}", c["batch"], c["L"], c["dim"], c["N"], c["io"], c["a_init"],
                        key=700 + seed, mode=mode)
    return c, wl


@pytest.mark.parametrize("seed", range(16))
def test_forward_random_shapes(seed):
    c, wl = _case(seed)
    announce(f"forward random seed={seed}: {c}")
    inp = datagen.scan_inputs(wl)
    t = upload_scan(inp, wl.io)
    h0 = datagen.gen_state(wl, "h0") if c["h0"] else None
    hs = torch.full((wl.batch, wl.dim, wl.dstate), float("nan"), device="cuda")
    y = sscan.forward(t["x"], t["delta"], t["A"], t["B"], t["C"], t["Dskip"] if c["skip"] else None,
                      final_state=hs, initial_state=None if h0 is None else torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    yr, hr = oracle.forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
                            inp["Dskip"] if c["skip"] else None, h0=h0, nthreads=oracle_threads())
    ey, eh = rel_err(to_host(y), yr), rel_err(hs.cpu().numpy(), hr)
    announce(f"  err(y)={ey:.2e} err(h)={eh:.2e}")
    assert ey <= TOL[wl.io] and eh <= TOL[wl.io], (ey, eh)


@pytest.mark.parametrize("seed", range(16, 26))
def test_backward_random_shapes(seed):
    c, wl = _case(seed)
    announce(f"backward random seed={seed}: {c}")
    inp = datagen.scan_inputs(wl)
    g = datagen.grad_inputs(wl)
    t = upload_scan(inp, wl.io)
    h0 = g["h0"] if c["h0"] else None
    dhT = g["dhT"] if c["dhT"] else None
    out = sscan.backward(t["x"], t["delta"], t["A"], t["B"], t["C"], to_dev(g["dy"], wl.io),
                         Dskip=t["Dskip"] if c["skip"] else None,
                         initial_state=None if h0 is None else torch.from_numpy(h0).cuda(),
                         dfinal_state=None if dhT is None else torch.from_numpy(dhT).cuda())
    torch.cuda.synchronize()
    ref = oracle.backward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
                          inp["Dskip"] if c["skip"] else None, g["dy"], h0, dhT, nthreads=oracle_threads())
    pairs = [("dx", "dx"), ("ddelta", "ddelta"), ("dA", "dA"), ("dB", "dB"), ("dC", "dC"),
             ("dinitial_state", "dh0")] + ([("dDskip", "dDskip")] if c["skip"] else [])
    errs = {k: rel_err(to_host(out[k]), ref[r]) for k, r in pairs}
    announce("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= TOL[wl.io], (k, e)


@pytest.mark.parametrize("seed", range(26, 34))
def test_scalar_A_random_shapes(seed):
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.choice([1, 2, 4]))
    H = G * int(rng.integers(1, 4))
    N = int(rng.choice([64, 128]))
    L = int(rng.choice([1, 63, 64, 65, 127, 129, int(rng.integers(2, 400))]))
    io = str(rng.choice(["f32", "bf16"]))
    wl = datagen.SsdWorkload(f"rssd{seed}", 800 + seed, int(rng.integers(1, 3)), L, H, 64, G, N, io)
    skip, with_h0 = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    announce(f"scalar-A random seed={seed}: b={wl.batch} L={L} H={H} G={G} N={N} io={io} "
             f"skip={skip} h0={with_h0}")
    inp = datagen.ssd_inputs(wl)
    h0 = (np.random.default_rng(seed).standard_normal((wl.batch, H, 64, N)).astype(np.float32)
          if with_h0 else None)
    up = lambda k: to_dev(inp[k], io)
    hs = torch.full((wl.batch, H, 64, N), float("nan"), device="cuda")
    y = sscan.ssd_forward(up("x"), up("delta"), torch.from_numpy(inp["A"]).cuda(), up("B"), up("C"),
                          torch.from_numpy(inp["D"]).cuda() if skip else None,
                          initial_state=None if h0 is None else torch.from_numpy(h0).cuda(), final_state=hs)
    torch.cuda.synchronize()
    yr, hr = oracle.ssd_forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                inp["D"] if skip else None, h0=h0)
    ey, eh = rel_err(to_host(y), yr), rel_err(hs.cpu().numpy(), hr)
    announce(f"  err(y)={ey:.2e} err(h)={eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io], (ey, eh)


@pytest.mark.parametrize("seed", range(34, 40))
def test_step_random_shapes(seed):
    c, wl = _case(seed, mode="step")
    steps = 12
    announce(f"step random seed={seed}: {c}")
    A, D = datagen.gen_A(wl), datagen.gen_Dskip(wl)
    bias = datagen.gen_dt_bias(wl)
    state0 = datagen.gen_state(wl, "h0")
    state = torch.from_numpy(state0).cuda()
    ref = state0.astype(np.float64)
    At, Dt = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    for k in range(steps):
        s = datagen.step_inputs(wl, k, bias=bias)
        yt = sscan.step(state, to_dev(s["x"], wl.io), to_dev(s["delta"], wl.io), At, to_dev(s["B"], wl.io),
                        to_dev(s["C"], wl.io), Dt if c["skip"] else None)
        torch.cuda.synchronize()
        yr, ref = oracle.step(ref, s["x"], s["delta"], A, s["B"], s["C"], D if c["skip"] else None)
        assert rel_err(to_host(yt), yr) <= TOL[wl.io], k
    e = rel_err(state.cpu().numpy(), ref)
    announce(f"  err(state)={e:.2e}")
    assert e <= TOL[wl.io], e
