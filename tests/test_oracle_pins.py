"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a
hand-worked exact example, the analytic or numerically integrated solution of
the continuous system, the convolution form of the time-invariant case, the
gated-EMA form of the one-dimensional selective update, limits and invariants,
or a brute-force unrolling.  Together they are chosen so that a dropped term,
a wrong sign or index, a transposed operand or Euler in place of ZOH fails at
least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand_problem(rng, batch, L, dim, N, a_lo=0.3, a_hi=3.0):
    x = rng.standard_normal((batch, L, dim))
    delta = np.exp(rng.uniform(np.log(1e-3), np.log(0.8), (batch, L, dim)))
    A = -rng.uniform(a_lo, a_hi, (dim, N))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    D = rng.standard_normal(dim)
    return x, delta, A, B, C, D


# ---------------------------------------------------------------- hand-worked exact examples

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    """Exact rational answers derived by hand from eq. (2) of 'The loop that beats attention'."""
    ln2 = math.log(2.0)
    arr = {k: np.array(case[k], dtype=np.float64) for k in ("x", "delta", "A", "B", "C", "Dskip")}
    for k in case["ln2_units"]:
        arr[k] = arr[k] * ln2
    y, hs = oracle.forward(arr["x"][None], arr["delta"][None], arr["A"], arr["B"][None],
                           arr["C"][None], arr["Dskip"])
    np.testing.assert_allclose(y[0], np.array(case["y"]), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(hs[0], np.array(case["final_state"]), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- ZOH == exact ODE solution

def _rk4_hold(a, h, u, T, steps):
    """Integrate h' = a*h + u over [0, T] with the input held constant (classical RK4)."""
    dt = T / steps
    for _ in range(steps):
        k1 = a * h + u
        k2 = a * (h + 0.5 * dt * k1) + u
        k3 = a * (h + 0.5 * dt * k2) + u
        k4 = a * (h + dt * k3) + u
        h = h + dt / 6.0 * (k1 + 2 * k2 + 2 * k3 + k4)
    return h


def test_zoh_step_equals_ode_integrated_with_held_input():
    """One discrete step lands where the continuous system does after delta with x held
    ('Mamba and State Space Models', Mechanism: zero-order hold). Pins the discretisation."""
    rng = np.random.default_rng(1)
    batch, L, dim, N = 1, 6, 3, 4
    x, delta, A, B, C, D = _rand_problem(rng, batch, L, dim, N)
    A[0, 1] = 0.0          # the A -> 0 limit
    A[1, 2] = 0.4          # a growing mode (eigenvalue above 1 after discretisation)
    _, hs_all = None, []
    for t in range(1, L + 1):
        _, hs = oracle.forward(x[:, :t], delta[:, :t], A, B[:, :t], C[:, :t], D)
        hs_all.append(hs[0])
    for d in range(dim):
        for n in range(N):
            h = 0.0
            for t in range(L):
                h = _rk4_hold(A[d, n], h, B[0, t, n] * x[0, t, d], delta[0, t, d], 400)
                assert abs(h - hs_all[t][d, n]) <= 1e-10 * max(1.0, abs(h)), (d, n, t)


def test_step_response_matches_analytic_ode_solution():
    """Constant input from rest: the continuous solution h(T) = (B x / -A)(1 - e^{A T}) is
    sampled exactly by ZOH at T = (t+1) * delta."""
    L, dim, N = 40, 2, 3
    A = np.array([[-0.5, -1.0, -3.0], [-0.1, -2.0, -0.7]])
    delta = np.full((1, L, dim), 0.05)
    x = np.full((1, L, dim), 1.7)
    B = np.tile(np.array([0.9, -1.3, 2.0]), (1, L, 1))
    C = np.zeros((1, L, N))
    _, hs = oracle.forward(x, delta, A, B, C, None)
    T = L * 0.05
    expect = (B[0, 0][None, :] * 1.7 / -A) * (1.0 - np.exp(A * T))
    np.testing.assert_allclose(hs[0], expect, rtol=1e-12)


# ---------------------------------------------------------------- GRU gate (1-D selective update)

def test_one_dimensional_update_is_the_gru_gate():
    """With N=1, A=-1, B=C=1 and delta=softplus(u) the ZOH update is the gated EMA
    h = (1 - sigmoid(u)) h + sigmoid(u) x ('Mamba matches the Transformer...', the gate
    interpretation under 'Selection makes the recurrence read the token').  An Euler
    discretisation (Bbar = delta*B) fails this."""
    rng = np.random.default_rng(2)
    L = 200
    u = rng.standard_normal(L) * 2.0
    xs = rng.standard_normal(L)
    delta = np.log1p(np.exp(u))
    y, _ = oracle.forward(xs[None, :, None], delta[None, :, None], np.array([[-1.0]]),
                          np.ones((1, L, 1)), np.ones((1, L, 1)), None)
    g = 1.0 / (1.0 + np.exp(-u))
    h, ref = 0.0, []
    for t in range(L):
        h = (1.0 - g[t]) * h + g[t] * xs[t]
        ref.append(h)
    np.testing.assert_allclose(y[0, :, 0], ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- time-invariant case == convolution

def _lti_problem(rng, L=64, dim=3, N=5):
    A = -rng.uniform(0.1, 2.0, (dim, N))
    dconst = rng.uniform(0.01, 0.5, dim)
    delta = np.broadcast_to(dconst, (1, L, dim)).copy()
    Bc, Cc = rng.standard_normal(N), rng.standard_normal(N)
    B = np.broadcast_to(Bc, (1, L, N)).copy()
    C = np.broadcast_to(Cc, (1, L, N)).copy()
    x = rng.standard_normal((1, L, dim))
    D = rng.standard_normal(dim)
    # kernel K_k = C Abar^k Bbar ('The loop that beats attention', eq. (3))
    Abar = np.exp(dconst[:, None] * A)
    Bbar = np.expm1(dconst[:, None] * A) / A * Bc[None, :]
    K = np.stack([(Cc[None, :] * Abar ** k * Bbar).sum(1) for k in range(L)])  # (L, dim)
    return x, delta, A, B, C, D, K


def test_time_invariant_case_equals_direct_convolution():
    rng = np.random.default_rng(3)
    x, delta, A, B, C, D, K = _lti_problem(rng)
    y, _ = oracle.forward(x, delta, A, B, C, D)
    L, dim = K.shape
    ref = np.zeros((L, dim))
    for t in range(L):
        for k in range(t + 1):
            ref[t] += K[k] * x[0, t - k]
    ref += D[None, :] * x[0]
    np.testing.assert_allclose(y[0], ref, rtol=1e-11, atol=1e-12)


def test_time_invariant_case_equals_fft_convolution():
    """Same case evaluated as a frequency-domain product ('Mamba and State Space Models',
    S4: a recurrence is also a convolution)."""
    rng = np.random.default_rng(4)
    x, delta, A, B, C, D, K = _lti_problem(rng, L=128)
    y, _ = oracle.forward(x, delta, A, B, C, D)
    L = K.shape[0]
    nfft = 2 * L
    ref = np.fft.irfft(np.fft.rfft(K, nfft, axis=0) * np.fft.rfft(x[0], nfft, axis=0), nfft, axis=0)[:L]
    ref += D[None, :] * x[0]
    np.testing.assert_allclose(y[0], ref, rtol=1e-9, atol=1e-11)


# ---------------------------------------------------------------- selective case: brute-force unroll

@pytest.mark.parametrize("seed", [5, 6, 7])
def test_brute_force_unrolled_sum(seed):
    """y_t = sum_{s<=t} sum_n C_t[n] (prod_{r=s+1..t} Abar_r[n]) Bbar_s[n] x_s + D x_t
    (the recurrence written out; time-varying Abar, Bbar after selection)."""
    rng = np.random.default_rng(seed)
    batch, L, dim, N = 2, 24, 3, 4
    x, delta, A, B, C, D = _rand_problem(rng, batch, L, dim, N)
    A[2, 3] = 0.0
    y, hs = oracle.forward(x, delta, A, B, C, D)
    for b in range(batch):
        for d in range(dim):
            Abar = np.exp(delta[b, :, d][:, None] * A[d][None, :])  # (L, N)
            with np.errstate(invalid="ignore", divide="ignore"):
                g = np.where(A[d] != 0, np.expm1(delta[b, :, d][:, None] * A[d]) / A[d],
                             delta[b, :, d][:, None])
            Bbar = g * B[b]
            for t in range(L):
                tot = D[d] * x[b, t, d]
                for s in range(t + 1):
                    prod = np.prod(Abar[s + 1:t + 1], axis=0) if s < t else np.ones(N)
                    tot += np.sum(C[b, t] * prod * Bbar[s]) * x[b, s, d]
                assert abs(tot - y[b, t, d]) <= 1e-11 * max(1.0, abs(tot))
            hL = sum(np.prod(Abar[s + 1:], axis=0) * Bbar[s] * x[b, s, d] for s in range(L))
            np.testing.assert_allclose(hs[b, d], hL, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- limits: forget and ignore

def test_large_delta_forgets_the_past():
    """Large delta drives Abar to 0: the state is overwritten by -B x / A and nothing before
    that token reaches later outputs ('Mamba and State Space Models', the selective state)."""
    rng = np.random.default_rng(8)
    batch, L, dim, N = 1, 30, 2, 3
    x, delta, A, B, C, D = _rand_problem(rng, batch, L, dim, N)
    t0 = 17
    delta[:, t0, :] = 1e4
    y1, h1 = oracle.forward(x, delta, A, B, C, D)
    x2, d2, B2 = x.copy(), delta.copy(), B.copy()
    x2[:, :t0] = rng.standard_normal(x2[:, :t0].shape)
    d2[:, :t0] *= 3.0
    B2[:, :t0] = rng.standard_normal(B2[:, :t0].shape)
    y2, h2 = oracle.forward(x2, d2, A, B2, C, D)
    assert not np.allclose(y1[:, :t0], y2[:, :t0])
    np.testing.assert_array_equal(y1[:, t0:], y2[:, t0:])
    np.testing.assert_array_equal(h1, h2)
    # state right after the reset token: h = -B x / A
    _, hr = oracle.forward(x[:, :t0 + 1], delta[:, :t0 + 1], A, B[:, :t0 + 1], C[:, :t0 + 1], D)
    np.testing.assert_allclose(hr[0], -B[0, t0][None, :] * x[0, t0][:, None] / A, rtol=1e-14)


def test_zero_delta_ignores_the_token():
    """delta = 0: Abar = 1, Bbar = 0, the state coasts and y_t = C_t h_{t-1} + D x_t."""
    rng = np.random.default_rng(9)
    batch, L, dim, N = 2, 12, 3, 4
    x, delta, A, B, C, D = _rand_problem(rng, batch, L, dim, N)
    t0 = 7
    delta[:, t0, :] = 0.0
    y, _ = oracle.forward(x, delta, A, B, C, D)
    _, hprev = oracle.forward(x[:, :t0], delta[:, :t0], A, B[:, :t0], C[:, :t0], D)
    _, hnow = oracle.forward(x[:, :t0 + 1], delta[:, :t0 + 1], A, B[:, :t0 + 1], C[:, :t0 + 1], D)
    np.testing.assert_array_equal(hnow, hprev)
    ref = np.einsum("bn,bdn->bd", C[:, t0], hprev) + D[None] * x[:, t0]
    np.testing.assert_allclose(y[:, t0], ref, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- associativity of the scan combine

def _fold(pairs):
    h = 0.0
    for a, b in pairs:
        h = a * h + b
    return h


def _combine(p, q):
    # (a1, b1) then (a2, b2): h -> a2 (a1 h + b1) + b2
    return (p[0] * q[0], q[0] * p[1] + q[1])


def _tree(pairs, splits):
    if len(pairs) == 1:
        return pairs[0]
    k = 1 + splits[0] % (len(pairs) - 1)
    rest = splits[1:] or [0]
    return _combine(_tree(pairs[:k], rest), _tree(pairs[k:], rest[::-1]))


@settings(max_examples=200, deadline=None)
@given(st.lists(st.tuples(st.floats(0.0, 1.0), st.floats(-3.0, 3.0)), min_size=1, max_size=40),
       st.lists(st.integers(0, 1000), min_size=1, max_size=8))
def test_any_bracketing_of_the_combine_equals_the_sequential_loop(pairs, splits):
    """The linear update composes associatively ('Mamba and State Space Models', the parallel
    scan; 'State space models and Mamba', associative scan), so any bracketing of
    (a1,b1)o(a2,b2) = (a1 a2, a2 b1 + b2) gives the sequential result."""
    a, b = _tree(pairs, splits)
    assert abs(b - _fold(pairs)) <= 1e-9 * max(1.0, sum(abs(q) for _, q in pairs))
    assert abs(a - np.prod([p for p, _ in pairs])) <= 1e-12


def test_combine_of_discretised_pairs_gives_the_oracle_state():
    rng = np.random.default_rng(10)
    L, N = 33, 3
    x, delta, A, B, C, D = _rand_problem(rng, 1, L, 1, N)
    _, hs = oracle.forward(x, delta, A, B, C, D)
    for n in range(N):
        a = np.exp(delta[0, :, 0] * A[0, n])
        bb = np.expm1(delta[0, :, 0] * A[0, n]) / A[0, n] * B[0, :, n] * x[0, :, 0]
        pairs = list(zip(a, bb))
        agg = _tree(pairs, [5, 11, 2, 7])
        assert abs(agg[1] - hs[0, 0, n]) <= 1e-12 * max(1.0, abs(hs[0, 0, n]))


# ---------------------------------------------------------------- constant state, resumability, step

def test_state_size_is_independent_of_length():
    rng = np.random.default_rng(11)
    for L in (1, 7, 300):
        x, delta, A, B, C, D = _rand_problem(rng, 2, L, 3, 4)
        _, hs = oracle.forward(x, delta, A, B, C, D)
        assert hs.shape == (2, 3, 4)


def test_split_sequence_resumes_from_the_snapshot():
    """forward([0,L)) == forward([0,L1)) then forward([L1,L)) from its final state
    ('Mamba and State Space Models', failure mode 2: snapshot and restore of the state)."""
    rng = np.random.default_rng(12)
    x, delta, A, B, C, D = _rand_problem(rng, 2, 50, 3, 4)
    y, hs = oracle.forward(x, delta, A, B, C, D)
    L1 = 19
    ya, ha = oracle.forward(x[:, :L1], delta[:, :L1], A, B[:, :L1], C[:, :L1], D)
    yb, hb = oracle.forward(x[:, L1:], delta[:, L1:], A, B[:, L1:], C[:, L1:], D, h0=ha)
    np.testing.assert_array_equal(np.concatenate([ya, yb], axis=1), y)
    np.testing.assert_array_equal(hb, hs)


def test_decode_steps_equal_the_forward_pass():
    """L single-token steps from a zero state reproduce the whole-sequence pass
    (recurrent inference, constant work per token)."""
    rng = np.random.default_rng(13)
    batch, L, dim, N = 3, 20, 4, 5
    x, delta, A, B, C, D = _rand_problem(rng, batch, L, dim, N)
    y, hs = oracle.forward(x, delta, A, B, C, D)
    state = np.zeros((batch, dim, N))
    for t in range(L):
        yt, state = oracle.step(state, x[:, t], delta[:, t], A, B[:, t], C[:, t], D)
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(state, hs)


def test_linear_in_x_and_causal():
    rng = np.random.default_rng(14)
    x, delta, A, B, C, D = _rand_problem(rng, 1, 40, 3, 4)
    x2 = rng.standard_normal(x.shape)
    y1, _ = oracle.forward(x, delta, A, B, C, D)
    y2, _ = oracle.forward(x2, delta, A, B, C, D)
    y12, _ = oracle.forward(2.0 * x - 0.5 * x2, delta, A, B, C, D)
    np.testing.assert_allclose(y12, 2.0 * y1 - 0.5 * y2, rtol=1e-11, atol=1e-12)
    t0 = 25
    x3, d3, B3, C3 = x.copy(), delta.copy(), B.copy(), C.copy()
    x3[:, t0:] += 1.0
    d3[:, t0:] *= 2.0
    B3[:, t0:] -= 0.5
    C3[:, t0:] += 0.5
    y3, _ = oracle.forward(x3, d3, A, B3, C3, D)
    np.testing.assert_array_equal(y3[:, :t0], y1[:, :t0])


def test_threads_do_not_change_the_result():
    rng = np.random.default_rng(15)
    x, delta, A, B, C, D = _rand_problem(rng, 3, 40, 7, 4)
    y1, h1 = oracle.forward(x, delta, A, B, C, D, nthreads=1)
    y4, h4 = oracle.forward(x, delta, A, B, C, D, nthreads=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(h1, h4)


def test_missing_skip_is_zero_skip():
    rng = np.random.default_rng(16)
    x, delta, A, B, C, D = _rand_problem(rng, 1, 10, 2, 3)
    y0, _ = oracle.forward(x, delta, A, B, C, None)
    yz, _ = oracle.forward(x, delta, A, B, C, np.zeros(2))
    np.testing.assert_array_equal(y0, yz)


# ---------------------------------------------------------------- backward pass

def _loss(inp, dy, dhT):
    y, hs = oracle.forward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"],
                           h0=inp["h0"])
    return float(np.sum(dy * y) + np.sum(dhT * hs))


def _grad_problem(seed):
    rng = np.random.default_rng(seed)
    batch, L, dim, N = 2, 7, 3, 3
    x, delta, A, B, C, D = _rand_problem(rng, batch, L, dim, N)
    A[1, 0] = 0.0            # the A -> 0 limit
    A[2, 2] = 0.3            # a growing mode
    inp = {"x": x, "delta": delta, "A": A, "B": B, "C": C, "Dskip": D,
           "h0": rng.standard_normal((batch, dim, N))}
    dy = rng.standard_normal((batch, L, dim))
    dhT = rng.standard_normal((batch, dim, N))
    return inp, dy, dhT


@pytest.mark.parametrize("seed", [21, 22])
def test_backward_matches_central_finite_differences(seed):
    """Every gradient against (L(p + e) - L(p - e)) / 2e of the forward oracle's scalar loss
    sum(dy * y) + sum(dhT * h_final); independent of how the backward pass is derived."""
    inp, dy, dhT = _grad_problem(seed)
    g = oracle.backward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"], dy,
                        h0=inp["h0"], dhT=dhT)
    names = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "Dskip": "dDskip",
             "h0": "dh0"}
    for key, gname in names.items():
        p = inp[key]
        num = np.zeros_like(p)
        for idx in np.ndindex(p.shape):
            eps = 1e-6 * max(1.0, abs(p[idx]))
            old = p[idx]
            p[idx] = old + eps
            lp = _loss(inp, dy, dhT)
            p[idx] = old - eps
            lm = _loss(inp, dy, dhT)
            p[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[gname], num, rtol=2e-6, atol=2e-7, err_msg=gname)


def test_backward_dx_is_the_transpose_of_the_linear_map():
    """With delta, B, C, A fixed and h0 = 0 the map x -> (y, h_final) is linear; the gradient
    dx for incoming (dy, dhT) must satisfy <dy, y(v)> + <dhT, h(v)> = <dx, v> for any v."""
    inp, dy, dhT = _grad_problem(23)
    g = oracle.backward(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"], dy,
                        dhT=dhT)
    rng = np.random.default_rng(24)
    for _ in range(3):
        v = rng.standard_normal(inp["x"].shape)
        y, hs = oracle.forward(v, inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"])
        lhs = np.sum(dy * y) + np.sum(dhT * hs)
        assert abs(lhs - np.sum(g["dx"] * v)) <= 1e-10 * max(1.0, abs(lhs))


def test_backward_is_linear_in_the_incoming_gradients_and_dD_is_closed_form():
    inp, dy, dhT = _grad_problem(25)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"])
    g1 = oracle.backward(*args, dy, h0=inp["h0"], dhT=dhT)
    g2 = oracle.backward(*args, 3.0 * dy, h0=inp["h0"], dhT=3.0 * dhT)
    for k in g1:
        np.testing.assert_allclose(g2[k], 3.0 * g1[k], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g1["dDskip"], np.einsum("bld,bld->d", dy, inp["x"]), rtol=1e-12)


def test_backward_threads_do_not_change_the_result():
    inp, dy, dhT = _grad_problem(26)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["Dskip"], dy)
    g1 = oracle.backward(*args, h0=inp["h0"], dhT=dhT, nthreads=1)
    g3 = oracle.backward(*args, h0=inp["h0"], dhT=dhT, nthreads=3)
    for k in g1:
        np.testing.assert_array_equal(g1[k], g3[k])


# ---------------------------------------------------------------- front end of the fused entry points
# The short causal convolution in front of the scan ("Mamba and State Space Models",
# "How this shows up in practice", d_conv) and delta = softplus(raw + bias) (the selective
# pseudocode).  Pinned against numpy routines and identities, not against its own formula.

def _fe_inputs(rng, batch=2, L=37, dim=5, K=4):
    return (rng.standard_normal((batch, L, dim)), rng.standard_normal((dim, K)),
            rng.standard_normal((batch, L, dim)) * 3.0, rng.standard_normal(dim),
            rng.standard_normal(dim), rng.standard_normal((batch, K - 1, dim)))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_frontend_conv_is_numpy_correlate_over_the_carried_inputs(K):
    rng = np.random.default_rng(40 + K)
    x, w, dr, cb, db, cs = _fe_inputs(rng, K=K)
    u, _, cs_out = oracle.frontend(x, w, dr, conv_bias=cb, delta_bias=db, act=0, conv_state=cs)
    for b in range(x.shape[0]):
        for d in range(x.shape[2]):
            seq = np.concatenate([cs[b, :, d], x[b, :, d]])
            ref = np.correlate(seq, w[d], mode="valid") + cb[d]
            np.testing.assert_allclose(u[b, :, d], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_array_equal(cs_out[b, :, d], seq[len(seq) - (K - 1):] if K > 1 else seq[:0])


def test_frontend_impulse_response_is_the_reversed_taps_and_zero_state_means_zeros():
    K, L, t0 = 4, 12, 5
    w = np.array([[0.5, -1.0, 2.0, 3.0]])
    x = np.zeros((1, L, 1)); x[0, t0, 0] = 1.0
    u, _, _ = oracle.frontend(x, w, np.zeros_like(x))
    expect = np.zeros(L)
    for j in range(K):
        expect[t0 + j] = w[0, K - 1 - j]   # tap K-1 sees the current token
    np.testing.assert_array_equal(u[0, :, 0], expect)
    # a unit carried input at row j (token j-(K-1)) reaches token 0 through tap j-... only
    cs = np.zeros((1, K - 1, 1)); cs[0, K - 2, 0] = 1.0   # the token just before 0
    u, _, _ = oracle.frontend(np.zeros((1, L, 1)), w, np.zeros((1, L, 1)), conv_state=cs)
    np.testing.assert_array_equal(u[0, :4, 0], [w[0, K - 2], w[0, K - 3], w[0, K - 4], 0.0])


def test_frontend_softplus_is_logaddexp():
    v = np.concatenate([np.linspace(-60, 60, 241), [0.0, 1e-300, -1e-300, 700.0, -700.0]])
    dr = v.reshape(1, -1, 1)
    _, delta, _ = oracle.frontend(np.zeros_like(dr), np.ones((1, 1)), dr)
    np.testing.assert_allclose(delta[0, :, 0], np.logaddexp(0.0, v), rtol=1e-14, atol=0)
    assert abs(delta[0, 241, 0] - np.log(2.0)) < 1e-16          # softplus(0) = ln 2
    # the bias is added before the softplus
    rng = np.random.default_rng(7)
    dr = rng.standard_normal((2, 9, 4)); db = rng.standard_normal(4)
    _, d1, _ = oracle.frontend(np.zeros_like(dr), np.ones((4, 1)), dr, delta_bias=db)
    np.testing.assert_allclose(d1, np.logaddexp(0.0, dr + db), rtol=1e-14)


def test_frontend_silu_reflection_and_zero():
    """silu(-c) = silu(c) - c (from sigmoid(-c) = 1 - sigmoid(c)); silu(0) = 0."""
    rng = np.random.default_rng(9)
    x, w, dr, _, _, cs = _fe_inputs(rng)
    c, _, _ = oracle.frontend(x, w, dr, act=0, conv_state=cs)
    up, _, _ = oracle.frontend(x, w, dr, act=1, conv_state=cs)
    un, _, _ = oracle.frontend(-x, w, dr, act=1, conv_state=-cs)
    np.testing.assert_allclose(un, up - c, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(up, c / (1.0 + np.exp(-c)), rtol=1e-13)   # against its definition
    z, _, _ = oracle.frontend(np.zeros_like(x), w, dr, act=1)
    assert not z.any()


def test_frontend_is_causal_and_streams_in_pieces():
    rng = np.random.default_rng(11)
    x, w, dr, cb, db, cs = _fe_inputs(rng, L=40)
    u, dl, cso = oracle.frontend(x, w, dr, cb, db, act=1, conv_state=cs)
    x2 = x.copy(); x2[:, 23, :] += 1.0
    u2, _, _ = oracle.frontend(x2, w, dr, cb, db, act=1, conv_state=cs)
    np.testing.assert_array_equal(u2[:, :23], u[:, :23])
    assert np.all(u2[:, 23] != u[:, 23])
    for L1 in (1, 2, 17):   # pieces shorter than the window too
        ua, da, csa = oracle.frontend(x[:, :L1], w, dr[:, :L1], cb, db, act=1, conv_state=cs)
        ub, db_, csb = oracle.frontend(x[:, L1:], w, dr[:, L1:], cb, db, act=1, conv_state=csa)
        np.testing.assert_array_equal(np.concatenate([ua, ub], axis=1), u)
        np.testing.assert_array_equal(np.concatenate([da, db_], axis=1), dl)
        np.testing.assert_array_equal(csb, cso)


def test_fused_forward_is_frontend_then_scan():
    rng = np.random.default_rng(13)
    x, w, dr, cb, db, cs = _fe_inputs(rng, L=30, dim=3)
    A = -np.exp(rng.uniform(-1, 1, (3, 4)))
    B, C = rng.standard_normal((2, 30, 4)), rng.standard_normal((2, 30, 4))
    D = rng.standard_normal(3)
    y, hs, cso = oracle.forward_fused(x, w, dr, A, B, C, D, cb, db, act=1, conv_state=cs)
    u = np.empty_like(x)
    for b in range(2):
        for d in range(3):
            c = np.correlate(np.concatenate([cs[b, :, d], x[b, :, d]]), w[d], "valid") + cb[d]
            u[b, :, d] = c / (1.0 + np.exp(-c))
    y2, hs2 = oracle.forward(u, np.logaddexp(0.0, dr + db), A, B, C, D)
    np.testing.assert_allclose(y, y2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(hs, hs2, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- scalar A per head (Mamba-2's SSM)
# The state space duality ("Mamba and State Space Models"; "Mamba matches the Transformer...",
# the duality section): with A a scalar per head the selective SSM is a lower-triangular,
# structured (semiseparable) matrix applied to x -- a masked "attention" whose score for
# (t, s) is C_t.B_s times the decay between s and t.

def _ssd_inputs(rng, batch=2, L=23, H=4, P=3, G=2, N=5, A_zero_head=False):
    x = rng.standard_normal((batch, L, H, P))
    delta = np.exp(rng.standard_normal((batch, L, H)) - 1.0)
    A = -np.exp(rng.standard_normal(H))
    if A_zero_head:
        A[1] = 0.0
    B = rng.standard_normal((batch, L, G, N))
    C = rng.standard_normal((batch, L, G, N))
    D = rng.standard_normal(H)
    return x, delta, A, B, C, D


def _ssd_dense(x, delta, A, B, C, D, h0=None):
    """y = M x + D x with M[t,s] = (C_t . B_s) exp(A (cum_t - cum_s)) gain_s for s <= t,
    cum the inclusive running sum of delta, gain_s = expm1(delta_s A)/A (delta_s at A = 0);
    plus, from an initial state, C_t . h0 exp(A cum_t)."""
    batch, L, H, P = x.shape
    G = B.shape[2]
    y = np.empty_like(x)
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            a = A[h]
            cum = np.cumsum(delta[b, :, h])
            gain = np.expm1(delta[b, :, h] * a) / a if a != 0 else delta[b, :, h]
            score = C[b, :, g] @ B[b, :, g].T                       # (L, L): C_t . B_s
            decay = np.exp(a * (cum[:, None] - cum[None, :]))
            M = np.tril(score * decay) * gain[None, :]
            y[b, :, h] = M @ x[b, :, h] + D[h] * x[b, :, h]
            if h0 is not None:
                y[b, :, h] += (C[b, :, g] @ h0[b, h].T) * np.exp(a * cum)[:, None]
    return y


@pytest.mark.parametrize("zero", [False, True])
def test_ssd_is_the_dense_semiseparable_matrix(zero):
    rng = np.random.default_rng(50 + zero)
    x, delta, A, B, C, D = _ssd_inputs(rng, A_zero_head=zero)
    y, _ = oracle.ssd_forward(x, delta, A, B, C, D)
    np.testing.assert_allclose(y, _ssd_dense(x, delta, A, B, C, D), rtol=1e-9, atol=1e-10)
    h0 = rng.standard_normal((2, 4, 3, 5))
    y, _ = oracle.ssd_forward(x, delta, A, B, C, D, h0=h0)
    np.testing.assert_allclose(y, _ssd_dense(x, delta, A, B, C, D, h0), rtol=1e-9, atol=1e-10)


def test_ssd_is_the_per_channel_scan_with_a_repeated_A():
    """One group: every (head, channel) is a channel of the per-channel scan whose A row is
    A_h repeated over the states and whose delta is the head's."""
    rng = np.random.default_rng(52)
    x, delta, A, B, C, D = _ssd_inputs(rng, G=1)
    batch, L, H, P = x.shape
    N = B.shape[3]
    h0 = rng.standard_normal((batch, H, P, N))
    y, hT = oracle.ssd_forward(x, delta, A, B, C, D, h0=h0)
    y2, hT2 = oracle.forward(x.reshape(batch, L, H * P), np.repeat(delta, P, axis=2),
                             np.repeat(A, P)[:, None] * np.ones((1, N)), B[:, :, 0], C[:, :, 0],
                             np.repeat(D, P), h0=h0.reshape(batch, H * P, N))
    np.testing.assert_allclose(y.reshape(batch, L, H * P), y2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hT.reshape(batch, H * P, N), hT2, rtol=1e-12, atol=1e-13)


def test_ssd_groups_share_B_and_C():
    rng = np.random.default_rng(53)
    x, delta, A, B, C, D = _ssd_inputs(rng, H=4, G=2)
    y, _ = oracle.ssd_forward(x, delta, A, B, C, D)
    # the same problem with one group per head, B/C replicated to each head of the group
    y1, _ = oracle.ssd_forward(x, delta, A, np.repeat(B, 2, axis=2), np.repeat(C, 2, axis=2), D)
    np.testing.assert_array_equal(y, y1)
    # a head reads only its own group: changing group 1 leaves heads 0-1 unchanged
    B2 = B.copy(); B2[:, :, 1] += 1.0
    y2, _ = oracle.ssd_forward(x, delta, A, B2, C, D)
    np.testing.assert_array_equal(y2[:, :, :2], y[:, :, :2])
    assert np.abs(y2[:, :, 2:] - y[:, :, 2:]).max() > 1e-3


def test_ssd_resumes_from_its_state():
    rng = np.random.default_rng(54)
    x, delta, A, B, C, D = _ssd_inputs(rng, L=30)
    y, hT = oracle.ssd_forward(x, delta, A, B, C, D)
    ya, ha = oracle.ssd_forward(x[:, :11], delta[:, :11], A, B[:, :11], C[:, :11], D)
    yb, hb = oracle.ssd_forward(x[:, 11:], delta[:, 11:], A, B[:, 11:], C[:, 11:], D, h0=ha)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hb, hT, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("nthreads", [2, 3, 7, 64])
def test_ssd_threads_do_not_change_the_result(nthreads):
    """Rows (batch row, head, channel) split over worker threads give the single-thread
    result bit for bit, with groups and an initial state (every row's loop is unchanged)."""
    rng = np.random.default_rng(55)
    x, delta, A, B, C, D = _ssd_inputs(rng, H=4, G=2, A_zero_head=True)
    h0 = rng.standard_normal((x.shape[0], 4, x.shape[3], B.shape[3]))
    y1, h1 = oracle.ssd_forward(x, delta, A, B, C, D, h0=h0, nthreads=1)
    yn, hn = oracle.ssd_forward(x, delta, A, B, C, D, h0=h0, nthreads=nthreads)
    np.testing.assert_array_equal(y1, yn)
    np.testing.assert_array_equal(h1, hn)
