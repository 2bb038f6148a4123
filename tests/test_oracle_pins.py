"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle's C loop against something other than itself:
a different form of the same method, a reduction to the Mamba-2 recurrence, a
closed form, an identity between SISO and MIMO, streaming schedules, or
invariants.  The last test plants mistakes in the oracle (its test hook) and
shows that the pins catch every one.
"""
import math

import numpy as np
import pytest

import oracle
from synth import custom, make_inputs, make_norm_params, make_state
from tests import pinforms as pf

TOL = 1e-11  # fp64 agreement, relative to rms(y)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    rms = math.sqrt(float(np.mean(b * b))) or 1.0
    return float(np.max(np.abs(a - b))) / rms if a.size else 0.0


def draw(**kw):
    w = custom(**kw)
    inp = make_inputs(w)
    return w, inp


def args_of(inp):
    return (inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"], inp["D"])


# ---------------------------------------------------------------- P1
@pytest.mark.parametrize("rank", [1, 3])
@pytest.mark.parametrize("bcnorm", [True, False])
def test_loop_equals_quadratic_form(rank, bcnorm):
    """P1: sequential loop == parallel form (L = S(alpha) @ Band) on T <= 16."""
    w, inp = draw(batch=2, seqlen=13, nheads=3, headdim=5, dstate=6, rank=rank, seed=11)
    # larger dt so the beta/gamma terms and the decay all matter
    inp["dt"] = (inp["dt"] * 8).astype(np.float32)
    npar = make_norm_params(w)
    gains = (npar["b_norm_w"], npar["c_norm_w"])
    biases = (npar["b_bias"], npar["c_bias"])
    y, _ = oracle.scan(*args_of(inp), bcnorm=bcnorm, b_norm_w=gains[0], c_norm_w=gains[1],
                       b_bias=biases[0], c_bias=biases[1])
    yq = pf.quadratic(*args_of(inp), bcnorm=bcnorm, gains=gains, biases=biases)
    assert rel_err(y, yq) < TOL


# ---------------------------------------------------------------- P2
def test_reduces_to_mamba2_at_lambda1_theta0():
    """P2: lambda = 1, theta = 0 gives the Mamba-2 recurrence and its dual form."""
    w, inp = draw(batch=2, seqlen=40, nheads=2, headdim=4, dstate=8, seed=5)
    inp["lam"] = np.ones_like(inp["lam"])
    inp["theta"] = np.zeros_like(inp["theta"])
    inp["dt"] = (inp["dt"] * 5).astype(np.float32)
    y, _ = oracle.scan(*args_of(inp), bcnorm=False)
    y2 = pf.mamba2_loop(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["D"])
    y2q = pf.mamba2_quadratic(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["D"])
    assert rel_err(y2, y2q) < TOL
    assert rel_err(y, y2) < TOL
    # with the norm on, against the Mamba-2 loop on normalised B, C
    y, _ = oracle.scan(*args_of(inp), bcnorm=True)
    assert rel_err(y, pf.mamba2_loop(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["D"],
                                     bcnorm=True)) < TOL


# ---------------------------------------------------------------- P3
@pytest.mark.parametrize("rank", [1, 2])
def test_rope_trick_equals_complex_state(rank):
    """P3: rotating B and C by the inclusive cumulative angle == complex diagonal state."""
    w, inp = draw(batch=1, seqlen=50, nheads=2, headdim=3, dstate=8, rank=rank, seed=9)
    inp["theta"] = (inp["theta"] * 4).astype(np.float32)  # angles up to pi/2 per step
    inp["dt"] = (inp["dt"] * 6).astype(np.float32)
    npar = make_norm_params(w)
    kw = dict(gains=(npar["b_norm_w"], npar["c_norm_w"]), biases=(npar["b_bias"], npar["c_bias"]))
    y, _ = oracle.scan(*args_of(inp), b_norm_w=kw["gains"][0], c_norm_w=kw["gains"][1],
                       b_bias=kw["biases"][0], c_bias=kw["biases"][1])
    yc = pf.complex_state_loop(*args_of(inp), **kw)
    assert rel_err(y, yc) < TOL


# ---------------------------------------------------------------- P4
@pytest.mark.parametrize("theta", [0.0, 0.2, 1.1])
@pytest.mark.parametrize("bcnorm", [False, True])
def test_closed_form(theta, bcnorm):
    """P4: constant coefficients, B = C = 1, x = 1: exact geometric-series output."""
    T, N, dt, A, lam = 60, 6, 0.3, -0.7, 0.35
    ones = np.ones((1, T, 1, N))
    x = np.ones((1, T, 1, 1))
    y, _ = oracle.scan(x, ones, ones, np.full((1, T, 1), dt), np.full((1, T, 1), lam),
                       np.full((1, T, 1, N // 2), theta), np.array([A]), np.array([0.0]),
                       bcnorm=bcnorm, eps=1e-5)
    ref = pf.closed_form(T, N, dt, A, lam, theta, eps=1e-5 if bcnorm else None)
    assert np.max(np.abs(y[0, :, 0, 0] - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_two_token_hand_derivation():
    """First two outputs written out by hand from the recurrence (not printed on the pages).

    B = C = 1 (norm off), x = 1, D = 0, constant dt, lambda, theta, zero state:
      y_0 = N lambda dt
      y_1 = N [ gamma (1 + alpha cos theta) + alpha dt (1 - lambda) cos theta ]
    (h_1 = alpha h_0 + beta B~_0 + gamma B~_1; each pair of C~_1 . B~_0 is 2 cos theta).
    """
    N, dt, A, lam, th = 6, 0.3, -0.7, 0.35, 0.2
    al, ga = math.exp(dt * A), lam * dt
    y0 = N * lam * dt
    y1 = N * (ga * (1 + al * math.cos(th)) + al * dt * (1 - lam) * math.cos(th))
    T = 2
    ones = np.ones((1, T, 1, N))
    y, _ = oracle.scan(np.ones((1, T, 1, 1)), ones, ones, np.full((1, T, 1), dt),
                       np.full((1, T, 1), lam), np.full((1, T, 1, N // 2), th), np.array([A]),
                       np.array([0.0]), bcnorm=False)
    assert abs(y[0, 0, 0, 0] - y0) < 1e-14 and abs(y[0, 1, 0, 0] - y1) < 1e-14
    assert abs(y0 - 0.63) < 1e-14 and abs(y1 - 2.0599677504) < 1e-9


# ---------------------------------------------------------------- P5
def test_mimo_rank1_is_siso():
    """P5a: MIMO with R = 1 is the SISO scan (rank axis squeezed)."""
    w, inp = draw(batch=2, seqlen=30, nheads=2, headdim=4, dstate=6, rank=1, seed=21)
    y, f = oracle.scan(*args_of(inp))
    ym, fm = oracle.scan(inp["x"][..., None], inp["B"][..., None], inp["C"][..., None],
                         *args_of(inp)[3:])
    assert rel_err(ym[..., 0], y) == 0.0
    assert rel_err(fm["h"], f["h"]) == 0.0


def test_mimo_is_sum_of_siso():
    """P5b: rank-R MIMO == R^2 SISO scans summed per output rank (D applied once per rank).

    torchmamba "Models" (MIMO: rank-R update on a shared state) and "Math notes"
    (MIMO training is R^2 SISO calls).
    """
    R = 3
    w, inp = draw(batch=1, seqlen=35, nheads=2, headdim=4, dstate=6, rank=R, seed=31)
    inp["dt"] = (inp["dt"] * 4).astype(np.float32)
    npar = make_norm_params(w)
    ym, _ = oracle.scan(*args_of(inp), b_norm_w=npar["b_norm_w"], c_norm_w=npar["c_norm_w"],
                        b_bias=npar["b_bias"], c_bias=npar["c_bias"])
    zero_D = np.zeros_like(inp["D"])
    ys = np.zeros_like(ym)
    for r in range(R):
        for rp in range(R):
            y, _ = oracle.scan(inp["x"][..., rp], inp["B"][..., rp], inp["C"][..., r],
                               *args_of(inp)[3:7], zero_D,
                               b_norm_w=npar["b_norm_w"], c_norm_w=npar["c_norm_w"],
                               b_bias=npar["b_bias"][:, rp:rp + 1], c_bias=npar["c_bias"][:, r:r + 1])
            ys[..., r] += y
        ys[..., r] += inp["D"].astype(np.float64)[None, None, :, None] * inp["x"][..., r].astype(np.float64)
    assert rel_err(ym, ys) < TOL


# ---------------------------------------------------------------- P6
@pytest.mark.parametrize("rank", [1, 2])
def test_streaming_schedules(rank):
    """P6: split schedules and token-by-token decode == one-shot, with the carried state.

    dotLLM PR #136 "Mamba-3 streaming decode" (split schedules reproduce
    one-shot once the previous B~ and x are carried); torchmamba "Quickstart"
    (forward == prefill + step).
    """
    w, inp = draw(batch=2, seqlen=17, nheads=2, headdim=3, dstate=4, rank=rank, seed=41)
    inp["dt"] = (inp["dt"] * 6).astype(np.float32)
    st0 = make_state(w, scale=0.5)
    full_y, full_f = oracle.scan(*args_of(inp), init=st0)
    for sched in ([9, 8], [2, 2, 2, 11], [1] * 17, [5, 1, 11], [16, 1]):
        st, ys, t0 = st0, [], 0
        for n in sched:
            part = {k: (v[:, t0:t0 + n] if k not in ("A", "D") else v) for k, v in inp.items()}
            y, st = oracle.scan(*args_of(part), init=st)
            ys.append(y)
            t0 += n
        assert rel_err(np.concatenate(ys, axis=1), full_y) < TOL
        for k in ("h", "prev_B", "prev_x", "angle"):
            assert rel_err(st[k], full_f[k]) < TOL, k


def test_empty_sequence_keeps_state():
    w, inp = draw(batch=1, seqlen=0, nheads=2, headdim=3, dstate=4, seed=3)
    st0 = make_state(w)
    y, f = oracle.scan(*args_of(inp), init=st0)
    assert y.shape == (1, 0, 2, 3)
    for k in ("h", "prev_B", "prev_x", "angle"):
        assert np.array_equal(f[k], st0[k].astype(np.float64))


# ---------------------------------------------------------------- P7
@pytest.mark.parametrize("Q", [1, 4, 16, 64, 100])
@pytest.mark.parametrize("rank", [1, 2])
def test_chunked_shifted_form_equals_loop(Q, rank):
    """P7: the chunkwise single-SSD form with the eta lookahead and local frames == loop.

    Also pins beta = alpha dt (1-lambda): the page's single-SSD fold (scale =
    gamma + dt_{t+1}(1-lambda_{t+1})) is exact only with that beta.
    """
    w, inp = draw(batch=1, seqlen=100, nheads=2, headdim=3, dstate=6, rank=rank, seed=51)
    inp["dt"] = (inp["dt"] * 5).astype(np.float32)
    st0 = make_state(w, scale=0.3)
    npar = make_norm_params(w)
    kw = dict(b_norm_w=npar["b_norm_w"], c_norm_w=npar["c_norm_w"],
              b_bias=npar["b_bias"], c_bias=npar["c_bias"])
    y, f = oracle.scan(*args_of(inp), init=st0, **kw)
    yc, fc = pf.chunked(*args_of(inp), Q, init=st0, gains=(kw["b_norm_w"], kw["c_norm_w"]),
                        biases=(kw["b_bias"], kw["c_bias"]))
    assert rel_err(yc, y) < 1e-10
    assert rel_err(fc["h"], f["h"]) < 1e-10
    assert rel_err(fc["prev_B"], f["prev_B"]) < 1e-10
    assert rel_err(fc["prev_x"], f["prev_x"]) == 0.0
    assert rel_err(fc["angle"], f["angle"]) < 1e-12


# ---------------------------------------------------------------- P8
def test_invariants():
    """P8: linearity in x, causality, and theta -> theta + 2 pi."""
    w, inp = draw(batch=1, seqlen=48, nheads=2, headdim=4, dstate=8, seed=61)
    y, _ = oracle.scan(*args_of(inp))
    rng = np.random.default_rng(0)
    x2 = rng.standard_normal(inp["x"].shape)
    y2, _ = oracle.scan(x2, *args_of(inp)[1:])
    y3, _ = oracle.scan(2.0 * inp["x"] - 3.0 * x2, *args_of(inp)[1:])
    assert rel_err(y3, 2.0 * y - 3.0 * y2) < TOL
    # causality: changing token 30 leaves outputs before it unchanged
    xp = inp["x"].copy()
    xp[:, 30] += 1.0
    Bp = inp["B"].copy()
    Bp[:, 30] -= 0.5
    yp, _ = oracle.scan(xp, Bp, *args_of(inp)[2:])
    assert np.array_equal(yp[:, :30], y[:, :30])
    assert not np.allclose(yp[:, 30:], y[:, 30:])
    # a full turn added to theta does not change y
    yt, _ = oracle.scan(*args_of(inp)[:5], inp["theta"].astype(np.float64) + 2 * np.pi, *args_of(inp)[6:])
    assert rel_err(yt, y) < 1e-11


# ---------------------------------------------------------------- planted mistakes
def _all_pins_pass(mutation):
    """Run a compact version of P1, P3, P4, P7 with the oracle's planted mistake."""
    w, inp = draw(batch=1, seqlen=12, nheads=2, headdim=3, dstate=6, seed=71)
    inp["dt"] = (inp["dt"] * 8).astype(np.float32)
    inp["theta"] = (inp["theta"] * 3).astype(np.float32)
    y, _ = oracle.scan(*args_of(inp), mutation=mutation)
    ok = rel_err(y, pf.quadratic(*args_of(inp))) < TOL
    ok &= rel_err(y, pf.complex_state_loop(*args_of(inp))) < TOL
    yc, _ = pf.chunked(*args_of(inp), 4)
    ok &= rel_err(y, yc) < 1e-10
    T, N = 20, 6
    ones = np.ones((1, T, 1, N))
    yf, _ = oracle.scan(np.ones((1, T, 1, 1)), ones, ones, np.full((1, T, 1), 0.3),
                        np.full((1, T, 1), 0.35), np.full((1, T, 1, N // 2), 0.2), np.array([-0.7]),
                        np.array([0.0]), bcnorm=False, mutation=mutation)
    ok &= np.max(np.abs(yf[0, :, 0, 0] - pf.closed_form(T, N, 0.3, -0.7, 0.35, 0.2))) < 1e-10
    return bool(ok)


def test_pins_catch_planted_mistakes():
    assert _all_pins_pass(0)
    # 1: beta without alpha; 2: exclusive angle sum; 3: rotation direction flipped;
    # 4: previous x paired with the current B~; 5: beta and gamma swapped
    for m in (1, 2, 3, 4, 5):
        assert not _all_pins_pass(m), f"planted mistake {m} not caught"
