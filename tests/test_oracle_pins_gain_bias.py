"""Property pins of the oracle's norm gains and biases on B and C (P17).

Mamba-3 block (torchmamba README, "Math notes"; dotLLM PR #136, "What lands here"):
B and C are RMS-normalised over N, scaled by a learned gain, offset by a learned
per-(head, rank) bias, then rotated by the cumulative data-dependent angle.  Two
properties fix where the gain and the bias act without restating the norm:

  (a) gain: a uniform gain c on B (no bias, D = 0, zero initial state) scales y, the
      final state h and prev_B by c; on C it scales y by c and leaves h unchanged.  A
      gain applied before the norm would cancel (y unchanged); a gain applied to the
      wrong operand moves the factor between y and h.
  (b) bias: raw B = 0 with bias b equals the un-normalised scan whose raw B is b
      broadcast over tokens (the bias is added before the rotation; a bias added
      after the rotation, or read as [H, N, R], gives another result).  Likewise C.
"""
import numpy as np
import pytest

import oracle
from synth import custom, make_inputs

TOL = 1e-11


def _case(R, seed=9):
    w = custom(batch=2, seqlen=29, nheads=3, headdim=5, dstate=8, rank=R, chunk=16, io="f32", seed=seed)
    inp = make_inputs(w)
    inp["D"] = np.zeros_like(inp["D"])
    return w, inp


def _run(inp, **kw):
    return oracle.scan(inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"], inp["D"], **kw)


def _rel(a, b):
    return float(np.abs(a - b).max() / (np.abs(b).max() or 1.0))


@pytest.mark.parametrize("R", [1, 3])
def test_uniform_gain_scales_state_part(R):
    w, inp = _case(R)
    N = w.dstate
    one = np.ones(N, np.float32)
    c = 1.75
    y1, f1 = _run(inp, b_norm_w=one, c_norm_w=one)
    yb, fb = _run(inp, b_norm_w=c * one, c_norm_w=one)
    yc, fc = _run(inp, b_norm_w=one, c_norm_w=c * one)
    assert np.abs(y1).max() > 1e-3
    assert _rel(yb, c * y1) < TOL and _rel(fb["h"], c * f1["h"]) < TOL and _rel(fb["prev_B"], c * f1["prev_B"]) < TOL
    assert _rel(yc, c * y1) < TOL and _rel(fc["h"], f1["h"]) < TOL and _rel(fc["prev_B"], f1["prev_B"]) < TOL


@pytest.mark.parametrize("R", [1, 2])
@pytest.mark.parametrize("which", ["B", "C"])
def test_bias_on_zero_input_is_unnormalised_input(R, which):
    w, inp = _case(R, seed=13)
    H, N = w.nheads, w.dstate
    eps = 1e-5
    bias = np.random.default_rng(5).standard_normal((H, R, N))
    other = "C" if which == "B" else "B"
    # The norm switch covers B and C together.  The other operand gets rows of mean square
    # 1 - eps, which the norm leaves unchanged (x / sqrt(1 - eps + eps) = x), so that the
    # normalised and the un-normalised runs see the same other operand.
    o = inp[other].astype(np.float64)
    o = o / np.sqrt(np.mean(o * o, axis=3, keepdims=True)) * np.sqrt(1.0 - eps)
    zero = dict(inp, **{which: np.zeros(inp[which].shape), other: o})
    y_b, f_b = _run(zero, bcnorm=True, eps=eps, **{("b_bias" if which == "B" else "c_bias"): bias})
    # un-normalised: the raw input is the bias broadcast over (batch, token), in the input's
    # [.., N] / [.., N, R] layout
    bt = np.transpose(bias, (0, 2, 1))  # [H, N, R]
    full = np.broadcast_to(bt if R > 1 else bt[..., 0], inp[which].shape)
    plain = dict(inp, **{which: np.ascontiguousarray(full), other: o})
    y_p, f_p = _run(plain, bcnorm=False)
    assert np.abs(y_p).max() > 1e-3
    assert _rel(y_b, y_p) < 1e-12
    assert _rel(f_b["h"], f_p["h"]) < 1e-12 and _rel(f_b["prev_B"], f_p["prev_B"]) < 1e-12


def test_bias_pin_catches_a_transposed_bias():
    """The bias read as [H, N, R] instead of [H, R, N] changes the result at R = 2 (N != R)."""
    w, inp = _case(2, seed=17)
    H, N, R = w.nheads, w.dstate, w.rank
    bias = np.random.default_rng(6).standard_normal((H, R, N)).astype(np.float32)
    wrong = np.ascontiguousarray(bias.reshape(H, N, R).transpose(0, 2, 1))
    zero = dict(inp)
    zero["B"] = np.zeros_like(inp["B"])
    y1, _ = _run(zero, b_bias=bias)
    y2, _ = _run(zero, b_bias=wrong)
    assert _rel(y1, y2) > 1e-3
