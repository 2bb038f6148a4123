"""Pins of the oracle's gradients (m3_oracle_bwd.c) by central finite differences.

The loss is L = sum(y * W) + sum over the final state of <final_k, V_k> with
random W, V; its gradient with respect to every input (and every element of
the initial state) from the reverse sweep is compared with
(L(v + e) - L(v - e)) / (2 e) computed from the forward oracle alone, in fp64.
Planted mistakes in the reverse sweep must fail the comparison.
"""
import math

import numpy as np
import pytest

import oracle
from synth import custom, make_block_inputs, make_inputs, make_norm_params, make_state

EPS = 1e-4  # central differences: truncation ~EPS^2, rounding ~1e-16 |L| / EPS
TOL = 1e-6  # relative to the rms of the gradient (finite-difference error here is ~1e-10 .. 5e-8)


def _loss(fwd_kw, W, V):
    y, fin = oracle.scan(**fwd_kw)
    L = float(np.sum(y * W))
    for k, v in V.items():
        L += float(np.sum(fin[k] * v))
    return L


def _case(rank=1, opts=False, bcnorm=True, T=7, N=6, P=3, H=2, Bsz=1, nr=2, seed=5, init=True):
    w = custom(batch=Bsz, seqlen=T, nheads=H, headdim=P, dstate=N, rank=rank, seed=seed)
    inp = {k: v.astype(np.float64) for k, v in make_inputs(w).items()}
    inp["dt"] = inp["dt"] * 10  # steps large enough for every term to matter
    inp["theta"] = inp["theta"] * 3
    npar = {k: v.astype(np.float64) for k, v in make_norm_params(w).items()}
    kw = dict(x=inp["x"], B=inp["B"], C=inp["C"], dt=inp["dt"], lam=inp["lam"], theta=inp["theta"],
              A=inp["A"], D=inp["D"], bcnorm=bcnorm, **npar)
    NR = N // 2
    if opts:
        ex = {k: v.astype(np.float64) for k, v in make_block_inputs(w, rope_pairs=nr).items()}
        kw.update(theta=ex["theta_p"] * 3, rope_pairs=nr, A=ex["A_tok"], dt=ex["dt_raw"] + 3.0,
                  dt_softplus=True, dt_bias=ex["dt_bias"], lam=ex["lam_raw"], lam_sigmoid=True, z=ex["z"])
        NR = nr
    if init:
        kw["init"] = {k: v.astype(np.float64) for k, v in make_state(w, scale=0.5, rope_pairs=NR).items()}
    rng = np.random.default_rng(seed + 100)
    W = rng.standard_normal(np.shape(kw["x"]))
    fin_shapes = dict(h=(Bsz, H, N, P), prev_B=(Bsz, H, N, rank), prev_x=(Bsz, H, P, rank), angle=(Bsz, H, NR))
    V = {k: rng.standard_normal(s) for k, s in fin_shapes.items()}
    return kw, W, V


def _analytic(kw, W, V, mutation=0):
    a = dict(kw)
    fwd = {k: a.pop(k) for k in ("x", "B", "C", "dt", "lam", "theta", "A", "D")}
    return oracle.scan_bwd(*fwd.values(), W, dfinal=V, mutation=mutation, **a)


def _fd_check(kw, W, V, g, names):
    worst = {}
    for name in names:
        if name.startswith("init."):
            key = name.split(".")[1]
            arr = kw["init"][key]
            an = g["init"][key]
        else:
            arr = kw[name]
            an = g[name]
        fd = np.zeros_like(arr)
        flat = arr.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + EPS
            lp = _loss(kw, W, V)
            flat[i] = old - EPS
            lm = _loss(kw, W, V)
            flat[i] = old
            fd.reshape(-1)[i] = (lp - lm) / (2 * EPS)
        rms = math.sqrt(float(np.mean(fd * fd))) or 1.0
        worst[name] = float(np.max(np.abs(np.asarray(an) - fd))) / rms
    return worst


CORE = ["x", "B", "C", "dt", "lam", "theta", "A", "D", "b_norm_w", "c_norm_w", "b_bias", "c_bias",
        "init.h", "init.prev_B", "init.prev_x", "init.angle"]


@pytest.mark.parametrize("rank", [1, 2])
def test_gradients_match_finite_differences(rank):
    kw, W, V = _case(rank=rank)
    g = _analytic(kw, W, V)
    worst = _fd_check(kw, W, V, g, CORE)
    assert all(v < TOL for v in worst.values()), worst


def test_gradients_norm_off():
    """Without the norm the gains have no effect (zero gradient) and B, C enter linearly."""
    kw, W, V = _case(bcnorm=False, seed=9)
    g = _analytic(kw, W, V)
    worst = _fd_check(kw, W, V, g, ["x", "B", "C", "dt", "theta", "b_bias", "c_bias", "b_norm_w"])
    assert all(v < TOL for v in worst.values() if v == v), worst
    assert np.all(g["b_norm_w"] == 0.0) and np.all(g["c_norm_w"] == 0.0)


@pytest.mark.parametrize("rank", [1, 2])
def test_gradients_with_every_option(rank):
    """Partial rotation, per-token A, softplus(dt + bias), sigmoid(lambda), silu(z) gate."""
    kw, W, V = _case(rank=rank, opts=True, seed=13)
    g = _analytic(kw, W, V)
    names = ["x", "B", "C", "dt", "lam", "theta", "A", "D", "dt_bias", "z", "b_bias", "c_norm_w",
             "init.h", "init.prev_B", "init.prev_x", "init.angle"]
    worst = _fd_check(kw, W, V, g, names)
    assert all(v < TOL for v in worst.values()), worst


@pytest.mark.parametrize("rank", [1, 2])
def test_gradients_half_split(rank):
    """Half-split pairing: the reverse sweep on the N-permuted problem equals finite
    differences of the forward loop, which pairs (i, i + N/2) natively."""
    kw, W, V = _case(rank=rank, seed=15 + rank)
    kw["half_split"] = True
    g = _analytic(kw, W, V)
    worst = _fd_check(kw, W, V, g, CORE)
    assert all(v < TOL for v in worst.values()), worst


def test_empty_sequence_passes_state_gradients():
    kw, W, V = _case(T=0, seed=3)
    g = _analytic(kw, W, V)
    for k in ("h", "prev_B", "prev_x", "angle"):
        assert np.array_equal(g["init"][k], V[k])
    assert g["x"].size == 0 and np.all(g["D"] == 0.0)


def test_planted_mistakes_are_caught():
    kw, W, V = _case(rank=1, seed=21)
    ok = lambda m: all(v < TOL for v in _fd_check(kw, W, V, _analytic(kw, W, V, m), ["dt", "theta", "B"]).values())
    assert ok(0)
    # 11: beta's dependence on dt dropped; 12: angle gradient sign; 13: norm factor held constant
    for m in (11, 12, 13):
        assert not ok(m), f"planted mistake {m} not caught"
