"""Pins of the oracle's canonical-block options against independent forms.

The options (partial rotation, per-token decay rate, softplus / sigmoid input
activations, silu output gate) are checked against the test-only quadratic and
complex-state forms of ``tests/pinforms.py``, against the Mamba-2 recurrence
where they reduce to it, and against streaming schedules.  The activations on
the reference side come from numpy / scipy routines, not from the oracle's C.
The last test plants the options' likely mistakes in the oracle and shows the
pins catch each one.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
from synth import custom, make_block_inputs, make_inputs, make_norm_params, make_state
from tests import pinforms as pf

TOL = 1e-11


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    rms = math.sqrt(float(np.mean(b * b))) or 1.0
    return float(np.max(np.abs(a - b))) / rms if a.size else 0.0


def softplus(v):
    return np.logaddexp(0.0, np.asarray(v, np.float64))


def draw(rope_pairs=None, **kw):
    w = custom(**kw)
    return w, make_inputs(w), make_block_inputs(w, rope_pairs=rope_pairs)


# ---------------------------------------------------------------- P9: per-token decay rate
@pytest.mark.parametrize("rank", [1, 2])
def test_per_token_A_equals_quadratic_and_complex(rank):
    """alpha_t = exp(dt_t A_t) with A per (batch, token, head).

    dotLLM PR #136, Stage D3 (per-(T,H) ADT from dd_A); the decay matrix of
    the parallel form is then the product of per-token alphas.
    """
    w, inp, ex = draw(batch=2, seqlen=13, nheads=2, headdim=3, dstate=6, rank=rank, seed=101)
    inp["dt"] = (inp["dt"] * 6).astype(np.float32)
    args = (inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], ex["A_tok"], inp["D"])
    y, _ = oracle.scan(*args)
    assert rel_err(y, pf.quadratic(*args)) < TOL
    assert rel_err(y, pf.complex_state_loop(*args)) < TOL
    # a per-token A that is constant over tokens is the per-head A
    Arep = np.broadcast_to(inp["A"][None, None, :], ex["A_tok"].shape).copy()
    y1, _ = oracle.scan(*args[:6], Arep, inp["D"])
    y2, _ = oracle.scan(*args[:6], inp["A"], inp["D"])
    assert rel_err(y1, y2) == 0.0


# ---------------------------------------------------------------- P10: partial rotation
@pytest.mark.parametrize("nr", [0, 1, 2, 3])
def test_partial_rotation_equals_quadratic_and_complex(nr):
    """Only the leading ``nr`` pairs rotate (dotLLM PR #136: num_rope_angles of d_state/2)."""
    w, inp, ex = draw(rope_pairs=nr, batch=1, seqlen=14, nheads=2, headdim=3, dstate=8, seed=103)
    th = (ex["theta_p"] * 4).astype(np.float32)
    inp["dt"] = (inp["dt"] * 6).astype(np.float32)
    args = (inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], th, inp["A"], inp["D"])
    y, f = oracle.scan(*args, rope_pairs=nr)
    assert f["angle"].shape == (1, 2, nr)
    assert rel_err(y, pf.quadratic(*args)) < TOL
    assert rel_err(y, pf.complex_state_loop(*args)) < TOL


def test_no_rotation_at_lambda1_is_mamba2():
    """rope_pairs = 0 and lambda = 1: the Mamba-2 recurrence (torchmamba "Models", reductions)."""
    w, inp, _ = draw(rope_pairs=0, batch=2, seqlen=40, nheads=2, headdim=4, dstate=8, seed=105)
    inp["dt"] = (inp["dt"] * 5).astype(np.float32)
    lam = np.ones_like(inp["lam"])
    th = np.zeros((2, 40, 2, 0), np.float32)
    y, _ = oracle.scan(inp["x"], inp["B"], inp["C"], inp["dt"], lam, th, inp["A"], inp["D"],
                       bcnorm=False, rope_pairs=0)
    assert rel_err(y, pf.mamba2_loop(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["D"])) < TOL


# ---------------------------------------------------------------- P11: input activations
@pytest.mark.parametrize("rank", [1, 2])
def test_input_activations(rank):
    """dt = softplus(dt_raw + dt_bias[h]), lambda = sigmoid(lam_raw) (dotLLM PR #136, Stage C)."""
    w, inp, ex = draw(batch=2, seqlen=12, nheads=3, headdim=3, dstate=6, rank=rank, seed=107)
    dt_raw = ex["dt_raw"] + 2.0  # larger steps so every term matters
    dt = softplus(dt_raw.astype(np.float64) + ex["dt_bias"].astype(np.float64)[None, None, :])
    lam = expit(ex["lam_raw"].astype(np.float64))
    npar = make_norm_params(w)
    kw = dict(b_norm_w=npar["b_norm_w"], c_norm_w=npar["c_norm_w"], b_bias=npar["b_bias"],
              c_bias=npar["c_bias"])
    y, _ = oracle.scan(inp["x"], inp["B"], inp["C"], dt_raw, ex["lam_raw"], inp["theta"], inp["A"],
                       inp["D"], dt_softplus=True, dt_bias=ex["dt_bias"], lam_sigmoid=True, **kw)
    ref = pf.quadratic(inp["x"], inp["B"], inp["C"], dt, lam, inp["theta"], inp["A"], inp["D"],
                       gains=(kw["b_norm_w"], kw["c_norm_w"]), biases=(kw["b_bias"], kw["c_bias"]))
    assert rel_err(y, ref) < TOL
    # no bias given = bias 0
    y0, _ = oracle.scan(inp["x"], inp["B"], inp["C"], dt_raw, inp["lam"], inp["theta"], inp["A"],
                        inp["D"], dt_softplus=True)
    ref0 = pf.quadratic(inp["x"], inp["B"], inp["C"], softplus(dt_raw), inp["lam"], inp["theta"],
                        inp["A"], inp["D"])
    assert rel_err(y0, ref0) < TOL


# ---------------------------------------------------------------- P12: output gate
@pytest.mark.parametrize("rank", [1, 3])
def test_output_gate(rank):
    """y = (C~^T h + D x) * silu(z), z laid out like y (dotLLM PR #136, Stage C)."""
    w, inp, ex = draw(batch=1, seqlen=11, nheads=2, headdim=4, dstate=6, rank=rank, seed=109)
    args = (inp["x"], inp["B"], inp["C"], inp["dt"] * 5, inp["lam"], inp["theta"], inp["A"], inp["D"])
    y, _ = oracle.scan(*args, z=ex["z"])
    z = ex["z"].astype(np.float64)
    assert rel_err(y, pf.quadratic(*args) * z * expit(z)) < TOL


# ---------------------------------------------------------------- P13: streaming with every option
@pytest.mark.parametrize("rank", [1, 2])
def test_streaming_with_options(rank):
    """Split schedules == one shot with partial rotation, per-token A, activations and gate.

    The carried angle holds only the rotated pairs; token 0 of a continued
    call activates its dt and lambda for the deferred boundary term (dotLLM
    PR #136, "Mamba-3 streaming decode").
    """
    nr = 2
    w, inp, ex = draw(rope_pairs=nr, batch=2, seqlen=15, nheads=2, headdim=3, dstate=8, rank=rank,
                      seed=111)
    full = dict(x=inp["x"], B=inp["B"], C=inp["C"], dt=ex["dt_raw"] + 2.0, lam=ex["lam_raw"],
                theta=ex["theta_p"] * 3, A=ex["A_tok"], z=ex["z"])
    opts = dict(rope_pairs=nr, dt_softplus=True, dt_bias=ex["dt_bias"], lam_sigmoid=True)
    st0 = make_state(w, scale=0.5, rope_pairs=nr)

    def run(part, init):
        return oracle.scan(part["x"], part["B"], part["C"], part["dt"], part["lam"], part["theta"],
                           part["A"], inp["D"], init=init, z=part["z"], **opts)

    full_y, full_f = run(full, st0)
    for sched in ([8, 7], [1] * 15, [3, 1, 11], [14, 1]):
        st, ys, t0 = st0, [], 0
        for n in sched:
            y, st = run({k: v[:, t0:t0 + n] for k, v in full.items()}, st)
            ys.append(y)
            t0 += n
        assert rel_err(np.concatenate(ys, axis=1), full_y) < TOL
        for k in ("h", "prev_B", "prev_x", "angle"):
            assert rel_err(st[k], full_f[k]) < TOL, k


# ---------------------------------------------------------------- P15: half-split pairing
@pytest.mark.parametrize("rank,nr", [(1, None), (2, None), (1, 2)])
def test_half_split_pairing_equals_complex_form(rank, nr):
    """Pair i made of components (i, i + N/2) (the rotate-half layout of the canonical block):
    the loop equals the complex-state form whose complex numbers are built from the two halves
    of N, with norm gains and biases and partial rotation; it differs from adjacent pairing."""
    w, inp, ex = draw(rope_pairs=nr, batch=2, seqlen=12, nheads=2, headdim=3, dstate=8, rank=rank, seed=117)
    inp["dt"] = (inp["dt"] * 6).astype(np.float32)
    th = (ex["theta_p"] if nr is not None else inp["theta"]) * 4
    args = (inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], th, inp["A"], inp["D"])
    prm = make_norm_params(w)
    kw = dict(rope_pairs=nr) if nr is not None else {}
    y, _ = oracle.scan(*args, half_split=True, **prm, **kw)
    ref = pf.complex_state_loop(*args, gains=(prm["b_norm_w"], prm["c_norm_w"]),
                                biases=(prm["b_bias"], prm["c_bias"]), half_split=True)
    assert rel_err(y, ref) < TOL
    y_adj, _ = oracle.scan(*args, **prm, **kw)
    assert rel_err(y_adj, ref) > 1e-3


def test_half_split_streaming():
    """Split schedules with the carried state (h and prev_B rows in the half-split layout)."""
    w, inp, ex = draw(batch=2, seqlen=11, nheads=2, headdim=3, dstate=8, rank=2, seed=119)
    full = {k: inp[k] for k in ("x", "B", "C", "dt", "lam", "theta")}
    st0 = make_state(w, scale=0.5)

    def run(part, init):
        return oracle.scan(part["x"], part["B"], part["C"], part["dt"], part["lam"], part["theta"],
                           inp["A"], inp["D"], init=init, half_split=True)

    full_y, full_f = run(full, st0)
    st, ys, t0 = st0, [], 0
    for n in (4, 1, 6):
        y, st = run({k: v[:, t0:t0 + n] for k, v in full.items()}, st)
        ys.append(y)
        t0 += n
    assert rel_err(np.concatenate(ys, axis=1), full_y) < TOL
    for k in ("h", "prev_B", "prev_x", "angle"):
        assert rel_err(st[k], full_f[k]) < TOL, k


# ---------------------------------------------------------------- planted mistakes
def _option_pins_pass(mutation):
    w, inp, ex = draw(rope_pairs=2, batch=1, seqlen=10, nheads=2, headdim=3, dstate=8, seed=113)
    inp["dt"] = (inp["dt"] * 6).astype(np.float32)
    th = (ex["theta_p"] * 4).astype(np.float32)
    args = (inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], th, ex["A_tok"], inp["D"])
    y, _ = oracle.scan(*args, rope_pairs=2, z=ex["z"], mutation=mutation)
    z = ex["z"].astype(np.float64)
    return rel_err(y, pf.quadratic(*args) * z * expit(z)) < TOL


def test_option_pins_catch_planted_mistakes():
    assert _option_pins_pass(0)
    # 6: A of the previous token; 7: the trailing pairs rotate; 8: sigmoid gate instead of silu
    for m in (6, 7, 8):
        assert not _option_pins_pass(m), f"planted mistake {m} not caught"
