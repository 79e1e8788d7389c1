"""GPU parity of sscan_forward against the fp64 oracle, through the C ABI.

Every named workload is compared element by element at full size: the tiny,
Mamba-130M and Mamba-1.4B widths in one oracle call each, and the 2^20-token
workload on every output of the whole sequence and its final state, with the
oracle run over 128-channel blocks of the device's own inputs (four tests of a
quarter of the channels each), plus a 4096-token prefix run.  Edge shapes cover L=1, ragged L and dim, every N, both A paths,
mixed A within a wave, A = 0 and A > 0, missing skip / final state, empty
inputs, non-finite propagation and run-to-run determinism.
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


def _run(t, wl, with_state=True, Dskip=True):
    hs = torch.full((wl.batch, wl.dim, wl.dstate), float("nan"), device="cuda") if with_state else None
    y = sscan.forward(t["x"], t["delta"], t["A"], t["B"], t["C"], t["Dskip"] if Dskip else None,
                      final_state=hs)
    torch.cuda.synchronize()
    return to_host(y), (hs.cpu().numpy() if with_state else None)


def _check_full(wl, seed=0, with_state=True, Dskip=True, inp=None):
    announce(f"forward {wl.name} b={wl.batch} L={wl.seqlen} dim={wl.dim} N={wl.dstate} io={wl.io}")
    inp = inp or datagen.scan_inputs(wl, seed)
    t = upload_scan(inp, wl.io)
    y, hs = _run(t, wl, with_state, Dskip)
    yr, hr = oracle.forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
                            inp["Dskip"] if Dskip else None, nthreads=oracle_threads(),
                            want_state=with_state)
    ey = rel_err(y, yr)
    eh = rel_err(hs, hr) if with_state else 0.0
    announce(f"  err(y)={ey:.3e} err(h)={eh:.3e}")
    assert ey <= TOL[wl.io], ey
    assert eh <= TOL[wl.io], eh
    return ey, eh


# ---------------------------------------------------------------- the named workloads

def test_tiny_f32_random_A():
    _check_full(datagen.workload("tiny_f32"))


def test_mamba130m_width_f32_full():
    _check_full(datagen.workload("mamba130m_f32"))


def test_mamba1p4b_width_bf16_full():
    """The benchmarked workload (4 x 8192 x 4096, N=16, bf16 I/O), every output checked."""
    _check_full(datagen.workload("mamba1p4b_bf16"))


@pytest.fixture(scope="module")
def long1m():
    """The 2^20-token x 2048-channel workload, run once on the GPU: inputs and outputs stay
    on the device for the checks below, which take the oracle over blocks of channels."""
    wl = datagen.workload("long1m_bf16")
    L, dim, N = wl.seqlen, wl.dim, wl.dstate
    announce(f"forward {wl.name}: generating {2 * L * dim / 1e9:.1f} G bf16 inputs")
    x = torch.empty(1, L, dim, dtype=torch.bfloat16, device="cuda")
    delta = torch.empty_like(x)
    span = 64 * datagen.TBLK
    for t0 in range(0, L, span):
        t1 = min(L, t0 + span)
        x[:, t0:t1] = to_dev(datagen.gen_seq(wl, "x", t0, t1), "bf16")
        delta[:, t0:t1] = to_dev(datagen.gen_seq(wl, "delta", t0, t1), "bf16")
    B = datagen.gen_seq(wl, "B")
    C = datagen.gen_seq(wl, "C")
    A = datagen.gen_A(wl)
    D = datagen.gen_Dskip(wl)
    hs = torch.full((1, dim, N), float("nan"), device="cuda")
    announce(f"forward {wl.name}: launching")
    y = sscan.forward(x, delta, torch.from_numpy(A).cuda(), to_dev(B, "bf16"), to_dev(C, "bf16"),
                      torch.from_numpy(D).cuda(), final_state=hs)
    torch.cuda.synchronize()
    yield {"wl": wl, "x": x, "delta": delta, "y": y, "hs": hs, "A": A, "B": B, "C": C, "D": D}
    del x, delta, y, hs
    torch.cuda.empty_cache()


def test_long_sequence_1m_tokens_prefix_every_channel(long1m):
    """Every output of the first 4096 tokens against an oracle run on that prefix."""
    t = long1m
    P = 4096
    yr, _ = oracle.forward(to_host(t["x"][:, :P]), to_host(t["delta"][:, :P]), t["A"], t["B"][:, :P],
                           t["C"][:, :P], t["D"], nthreads=oracle_threads(), want_state=False)
    e = rel_err(to_host(t["y"][:, :P]), yr)
    announce(f"  prefix err={e:.3e}")
    assert e <= TOL["bf16"], e


@pytest.mark.timeout(900)
@pytest.mark.parametrize("quarter", range(4))
def test_long_sequence_1m_tokens_every_output_and_final_state(long1m, quarter):
    """Every output of the whole 2^20-token sequence and the final state, a quarter of the
    2048 channels per test, against the oracle's sequential loop over the whole sequence
    (channels are independent, so the oracle runs on 128-channel blocks of the device's
    own bf16 inputs)."""
    t = long1m
    dim = t["wl"].dim
    q0, q1 = quarter * dim // 4, (quarter + 1) * dim // 4
    ey = eh = 0.0
    for c0 in range(q0, q1, 128):
        c1 = min(q1, c0 + 128)
        xb = to_host(t["x"][:, :, c0:c1].contiguous())
        db = to_host(t["delta"][:, :, c0:c1].contiguous())
        yr, hr = oracle.forward(xb, db, t["A"][c0:c1], t["B"], t["C"], t["D"][c0:c1],
                                nthreads=oracle_threads())
        del xb, db
        ey = max(ey, rel_err(to_host(t["y"][:, :, c0:c1].contiguous()), yr))
        eh = max(eh, rel_err(t["hs"][:, c0:c1].cpu().numpy(), hr))
        del yr
        announce(f"  channels [{c0},{c1}): err(y) so far={ey:.3e} err(h) so far={eh:.3e}")
    assert ey <= TOL["bf16"], ey
    assert eh <= TOL["bf16"], eh


# ---------------------------------------------------------------- edge shapes

EDGE = [
    # (batch, L, dim, N, io, a_init)
    (1, 1, 64, 16, "f32", "s4d_real"),
    (1, 1, 5, 3, "f32", "loguniform"),
    (2, 777, 100, 16, "f32", "s4d_real"),
    (2, 777, 100, 16, "bf16", "loguniform"),
    (3, 129, 65, 1, "f32", "loguniform"),
    (3, 129, 65, 1, "f32", "s4d_real"),
    (1, 300, 33, 2, "bf16", "s4d_real"),
    (1, 513, 70, 5, "f32", "s4d_real"),
    (2, 400, 130, 8, "f32", "loguniform"),
    (1, 20000, 64, 16, "f32", "s4d_real"),   # one tile: ~300 time segments
    (1, 9000, 7, 4, "bf16", "loguniform"),
    # >= 192 tiles of 64 channels: the lockstep kernel (ragged dim, N < 16, L = 1,
    # partial last chunk, exactly one chunk)
    (128, 300, 65, 16, "bf16", "s4d_real"),
    (200, 517, 64, 5, "f32", "s4d_real"),
    (200, 1, 64, 16, "f32", "s4d_real"),
    (64, 2100, 130, 8, "f32", "s4d_real"),
    (193, 700, 64, 1, "bf16", "s4d_real"),
    (256, 256, 64, 16, "f32", "s4d_real"),
    (192, 1000, 64, 2, "bf16", "s4d_real"),
    # 64..191 tiles: segment kernels
    (160, 517, 64, 5, "f32", "s4d_real"),
    (129, 700, 64, 1, "bf16", "s4d_real"),
]


@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "b{}_L{}_d{}_N{}_{}_{}".format(*s))
def test_edge_shapes(shape):
    batch, L, dim, N, io, a_init = shape
    wl = datagen.custom(f"edge_{batch}_{L}_{dim}_{N}_{io}_{a_init}", batch, L, dim, N, io, a_init, key=7)
    _check_full(wl)


def test_without_skip_and_without_final_state():
    wl = datagen.custom("noskip", 2, 300, 96, 16, "f32", "s4d_real", key=8)
    _check_full(wl, with_state=False, Dskip=False)


def test_mixed_A_within_a_wave_takes_the_general_path():
    """Channels 0..31 of the wave S4D-real, 32..63 random: the whole wave must still match."""
    wl = datagen.custom("mixed", 2, 500, 64, 16, "f32", "s4d_real", key=9)
    inp = datagen.scan_inputs(wl)
    rnd = datagen.gen_A(datagen.custom("mixedA", 1, 1, 64, 16, "f32", "loguniform", key=9))
    inp["A"] = np.concatenate([inp["A"][:32], rnd[32:]]).astype(np.float32)
    _check_full(wl, inp=inp)


def test_lockstep_with_some_general_tiles():
    """256 tiles: d-tile 1 and one channel of d-tile 6 have random A (segment kernels), the rest
    are S4D-real (lockstep kernel)."""
    wl = datagen.custom("mixedlock", 4, 1000, 4096, 16, "bf16", "s4d_real", key=15)
    inp = datagen.scan_inputs(wl)
    rnd = datagen.gen_A(datagen.custom("mixedlockA", 1, 1, 4096, 16, "f32", "loguniform", key=15))
    A = inp["A"].copy()
    A[64:128] = rnd[64:128]
    A[70 * 64 - 4096 + 5] = rnd[70 * 64 - 4096 + 5]
    inp["A"] = A
    _check_full(wl, inp=inp)


def test_zero_and_positive_A():
    """A = 0 (Bbar -> delta*B limit) and small A > 0 (growing mode) per channel."""
    wl = datagen.custom("zeroA", 1, 200, 70, 4, "f32", "loguniform", key=10)
    inp = datagen.scan_inputs(wl)
    A = inp["A"].copy()
    A[3, :] = 0.0
    A[5, 1] = 0.0
    A[9, :] = 0.05
    A[10, 2] = 0.2
    inp["A"] = A
    _check_full(wl, inp=inp)


def test_s4d_scaled_rows_take_the_fast_path_correctly():
    """A[d,n] = (n+1)*A[d,0] with a different A[d,0] per channel."""
    wl = datagen.custom("s4dscaled", 2, 1000, 128, 16, "bf16", "s4d_real", key=11)
    inp = datagen.scan_inputs(wl)
    scale = np.linspace(0.1, 3.0, 128, dtype=np.float32)[:, None]
    inp["A"] = (inp["A"] * scale).astype(np.float32)
    _check_full(wl, inp=inp)


def _slow_memory_inputs(wl, scales):
    """Small steps (delta ~ 1e-3, the low end of a usual dt range) and per-channel
    A scales down to 1e-4: delta*A is tiny, each token moves the state very little
    and the state integrates thousands of tokens.  fp32 must keep full precision
    there (a formulation whose rounding is relative to B*x rather than to the
    state loses about two digits)."""
    inp = datagen.scan_inputs(wl)
    rng = np.random.default_rng(17)
    inp["delta"] = (1e-3 * np.exp(0.5 * rng.standard_normal(inp["delta"].shape))).astype(np.float32)
    inp["A"] = (inp["A"] * scales[:, None]).astype(np.float32)
    return inp


@pytest.mark.parametrize("batch", [1, 256])  # segment kernels / lockstep kernel
def test_small_delta_times_A_keeps_fp32_precision(batch):
    wl = datagen.custom("slowmem", batch, 2048 if batch == 1 else 600, 128, 16, "f32", "s4d_real", key=12)
    scales = np.geomspace(1e-4, 1.0, 128).astype(np.float32)
    _check_full(wl, inp=_slow_memory_inputs(wl, scales))


def test_empty_inputs():
    dev = "cuda"
    x = torch.empty(1, 0, 8, device=dev)
    hs = torch.full((1, 8, 4), 7.0, device=dev)
    y = sscan.forward(x, x.clone(), torch.zeros(8, 4, device=dev), torch.empty(1, 0, 4, device=dev),
                      torch.empty(1, 0, 4, device=dev), final_state=hs)
    torch.cuda.synchronize()
    assert y.shape == (1, 0, 8)
    assert torch.all(hs == 0)
    z = torch.empty(0, 5, 8, device=dev)
    sscan.forward(z, z.clone(), torch.zeros(8, 4, device=dev), torch.empty(0, 5, 4, device=dev),
                  torch.empty(0, 5, 4, device=dev))
    torch.cuda.synchronize()


def test_non_finite_inputs_propagate_like_the_oracle():
    wl = datagen.custom("nan", 1, 200, 64, 16, "f32", "s4d_real", key=12)
    inp = datagen.scan_inputs(wl)
    inp["x"][0, 50, 3] = np.nan
    inp["delta"][0, 120, 7] = np.inf
    t = upload_scan(inp, "f32")
    y, hs = _run(t, wl)
    yr, hr = oracle.forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"])
    np.testing.assert_array_equal(np.isnan(y), np.isnan(yr))
    np.testing.assert_array_equal(np.isnan(hs), np.isnan(hr))
    ok = np.isfinite(yr)
    assert rel_err(y[ok], yr[ok]) <= TOL["f32"]


@pytest.mark.parametrize("a_init", ["s4d_real", "loguniform"])
def test_infinite_input_makes_its_channel_non_finite_like_the_oracle(a_init):
    """An infinite x makes the channel's state infinite from that token on.  The oracle's
    update Abar h + Bbar x keeps +-Inf; the structured-real update k + q (w - k) gives
    Inf - Inf = NaN on the next token (a state that is not finite either way), so what is
    compared is where the results are finite, and the finite values."""
    wl = datagen.custom("inf", 1, 400, 64, 16, "f32", a_init, key=18)
    inp = datagen.scan_inputs(wl)
    inp["x"][0, 150, 3] = np.inf
    t = upload_scan(inp, "f32")
    y, hs = _run(t, wl)
    yr, hr = oracle.forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"])
    np.testing.assert_array_equal(np.isfinite(y), np.isfinite(yr))
    np.testing.assert_array_equal(np.isfinite(hs), np.isfinite(hr))
    assert not np.isfinite(yr[0, 150:, 3]).any() and np.isfinite(yr[0, :150, 3]).all()
    ok = np.isfinite(yr)
    assert rel_err(y[ok], yr[ok]) <= TOL["f32"]


def test_run_to_run_bitwise_determinism():
    wl = datagen.custom("det", 2, 3000, 256, 16, "bf16", "s4d_real", key=13)
    t = upload_scan(datagen.scan_inputs(wl), "bf16")
    y1, h1 = _run(t, wl)
    y2, h2 = _run(t, wl)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(h1, h2)


def test_runs_on_a_side_stream():
    wl = datagen.custom("stream", 1, 1000, 128, 16, "f32", "s4d_real", key=14)
    inp = datagen.scan_inputs(wl)
    t = upload_scan(inp, "f32")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = sscan.forward(t["x"], t["delta"], t["A"], t["B"], t["C"], t["Dskip"])
    s.synchronize()
    yr, _ = oracle.forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"],
                           want_state=False)
    assert rel_err(to_host(y), yr) <= TOL["f32"]


# ---------------------------------------------------------------- starting from a state

STATE_SHAPES = [
    (2, 700, 100, 16, "f32", "s4d_real"),     # segment kernels, structured-real A
    (2, 700, 100, 8, "bf16", "loguniform"),   # segment kernels, general A
    (256, 300, 64, 16, "bf16", "s4d_real"),   # lockstep kernel
    (1, 20000, 64, 16, "f32", "s4d_real"),    # ~300 segments
    # segment counts that leave groups of the carry kernel (16 per workgroup) partly
    # filled or empty: 17 segments (groups of 2: nine used), 33 (groups of 3: eleven)
    (2, 64 * 17, 96, 16, "f32", "s4d_real"),
    (3, 64 * 33 + 5, 130, 16, "bf16", "loguniform"),
]


@pytest.mark.parametrize("shape", STATE_SHAPES, ids=lambda s: "b{}_L{}_d{}_N{}_{}_{}".format(*s))
def test_initial_state_matches_oracle(shape):
    batch, L, dim, N, io, a_init = shape
    wl = datagen.custom(f"h0_{batch}_{L}_{dim}_{N}_{io}", batch, L, dim, N, io, a_init, key=30)
    inp = datagen.scan_inputs(wl)
    h0 = (np.random.default_rng(5).standard_normal((batch, dim, N)) * 0.5).astype(np.float32)
    announce(f"forward_from_state {wl.name}")
    t = upload_scan(inp, io)
    hs = torch.full((batch, dim, N), float("nan"), device="cuda")
    y = sscan.forward(t["x"], t["delta"], t["A"], t["B"], t["C"], t["Dskip"], final_state=hs,
                      initial_state=torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    yr, hr = oracle.forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"], h0=h0,
                            nthreads=oracle_threads())
    ey, eh = rel_err(to_host(y), yr), rel_err(hs.cpu().numpy(), hr)
    announce(f"  err(y)={ey:.3e} err(h)={eh:.3e}")
    assert ey <= TOL[io] and eh <= TOL[io]


@pytest.mark.parametrize("shape", STATE_SHAPES[:3], ids=lambda s: "b{}_L{}_d{}_N{}_{}_{}".format(*s))
def test_prefill_in_two_pieces_equals_one_pass(shape):
    """forward over [0, L1), then forward_from_state over [L1, L) from its final state, against the
    oracle over [0, L) in one pass."""
    batch, L, dim, N, io, a_init = shape
    wl = datagen.custom(f"split_{batch}_{L}_{dim}_{N}_{io}", batch, L, dim, N, io, a_init, key=31)
    inp = datagen.scan_inputs(wl)
    L1 = 257
    dev = lambda a: to_dev(np.ascontiguousarray(a), io)
    A, D = torch.from_numpy(inp["A"]).cuda(), torch.from_numpy(inp["Dskip"]).cuda()
    h1 = torch.empty(batch, dim, N, device="cuda")
    h2 = torch.empty(batch, dim, N, device="cuda")
    ya = sscan.forward(dev(inp["x"][:, :L1]), dev(inp["delta"][:, :L1]), A, dev(inp["B"][:, :L1]),
                       dev(inp["C"][:, :L1]), D, final_state=h1)
    yb = sscan.forward(dev(inp["x"][:, L1:]), dev(inp["delta"][:, L1:]), A, dev(inp["B"][:, L1:]),
                       dev(inp["C"][:, L1:]), D, final_state=h2, initial_state=h1)
    torch.cuda.synchronize()
    yr, hr = oracle.forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"],
                            nthreads=oracle_threads())
    y = np.concatenate([to_host(ya), to_host(yb)], axis=1)
    assert rel_err(y, yr) <= TOL[io]
    assert rel_err(h2.cpu().numpy(), hr) <= TOL[io]


def test_empty_sequence_copies_the_initial_state():
    h0 = torch.randn(2, 8, 4, device="cuda")
    hs = torch.zeros(2, 8, 4, device="cuda")
    x = torch.empty(2, 0, 8, device="cuda")
    sscan.forward(x, x.clone(), torch.zeros(8, 4, device="cuda"), torch.empty(2, 0, 4, device="cuda"),
                  torch.empty(2, 0, 4, device="cuda"), final_state=hs, initial_state=h0)
    torch.cuda.synchronize()
    assert torch.equal(hs, h0)
