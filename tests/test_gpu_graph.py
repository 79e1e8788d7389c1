"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A serving loop launches the single-token step thousands of times; capturing a run of
steps once and replaying it removes the per-call host cost.  sscan_step and
sscan_step_fused enqueue one kernel each and allocate nothing, so they capture as
plain kernel nodes.  Each test runs the same steps eagerly, then replays the captured
steps three times from the same starting state, with eager work on the device between
the replays, and requires every replay to equal the eager run bit for bit (same
kernels, same inputs).
"""
import numpy as np
import pytest
import torch

import datagen
from tests.gpuutil import announce, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import selective_state_space_77_amd as sscan  # noqa: E402

STEPS = 8


def _staged(wl):
    bias = datagen.gen_dt_bias(wl)
    ins = [datagen.step_inputs(wl, k, bias=bias) for k in range(STEPS)]
    t = {k: torch.stack([to_dev(s[k], wl.io) for s in ins]) for k in ("x", "delta", "B", "C")}
    t["A"] = torch.from_numpy(datagen.gen_A(wl)).cuda()
    t["D"] = torch.from_numpy(datagen.gen_Dskip(wl)).cuda()
    t["state0"] = torch.from_numpy(datagen.gen_state(wl, "h0")).cuda()
    return t


def _replays_match(run, state0, state, outs, extra=()):
    """run(k) enqueues step k on the current stream; state, outs (and extra buffers,
    given with their starting values) are what the steps write."""
    state.copy_(state0)
    for buf, start in extra:
        buf.copy_(start)
    for k in range(STEPS):
        run(k)
    torch.cuda.synchronize()
    ref = [state.clone(), outs.clone()] + [buf.clone() for buf, _ in extra]

    state.copy_(state0)
    for buf, start in extra:
        buf.copy_(start)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(STEPS):
            run(k)
    for rep in range(3):
        # eager device work between replays: reset the written buffers
        state.copy_(state0)
        outs.zero_()
        for buf, start in extra:
            buf.copy_(start)
        g.replay()
        torch.cuda.synchronize()
        got = [state, outs] + [buf for buf, _ in extra]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (rep, i)
        announce(f"  replay {rep}: equal to the eager steps")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decode_steps_replay_from_a_graph(io):
    wl = datagen.custom(f"graph_step_{io}", 8, STEPS, 300, 16, io, "s4d_real", key=90, mode="step")
    announce(f"graph replay of {STEPS} decode steps, batch {wl.batch} x dim {wl.dim}, {io}")
    t = _staged(wl)
    state = torch.empty_like(t["state0"])
    Y = torch.empty_like(t["x"])

    def run(k):
        sscan.step(state, t["x"][k], t["delta"][k], t["A"], t["B"][k], t["C"][k], t["D"], y_t=Y[k])

    _replays_match(run, t["state0"], state, Y)


def test_fused_decode_steps_replay_from_a_graph():
    wl = datagen.custom("graph_step_fused", 8, STEPS, 300, 16, "bf16", "s4d_real", key=91, mode="step")
    K = 4
    announce(f"graph replay of {STEPS} fused decode steps (d_conv {K}, SiLU)")
    t = _staged(wl)
    fe = datagen.frontend_inputs(datagen.custom("graph_fe", 8, 1, 300, 16, "bf16", "s4d_real", key=91), K)
    w = torch.from_numpy(fe["conv_w"]).cuda()
    cb = torch.from_numpy(fe["conv_b"]).cuda()
    db = torch.from_numpy(fe["delta_bias"]).cuda()
    cs0 = to_dev(fe["conv_state"], "bf16")
    cs = torch.empty_like(cs0)
    state = torch.empty_like(t["state0"])
    Y = torch.empty_like(t["x"])

    def run(k):
        sscan.step_fused(state, cs, t["x"][k], w, t["delta"][k], t["A"], t["B"][k], t["C"][k], t["D"],
                         conv_bias=cb, delta_bias=db, activation="silu", y_t=Y[k])

    _replays_match(run, t["state0"], state, Y, extra=[(cs, cs0)])
