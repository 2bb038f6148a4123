"""Pins of the oracle's MIMO projections by learned per-rank vectors (P16).

torchmamba README, "Math notes", MIMO paragraph: the per-head x, z and y of the MIMO
block are expanded (x, z) and contracted (y) by learned per-rank vectors (D P + P R
parameters, not D P R); dotLLM PR #136, "What's deferred" (MIMO-in-Block: the mimo_x /
mimo_z projections and the post-scan rank contraction).  The projections are
elementwise, so the scan with them equals the plain MIMO scan (pinned by P5 against R
summed SISO scans) on inputs expanded, and outputs contracted, here with numpy:

  (a) rank 1 with unit vectors is the SISO scan;
  (b) mimo_x: the MIMO scan of x_r[p] = x[p] w_x[h, r, p];
  (c) mimo_o: sum_r w_o[h, r, p] y_r[p] of the MIMO scan's per-rank outputs;
  (d) mimo_z: the MIMO scan gated by z_r[p] = z[p] w_z[h, r, p];
  (e) all three, split into a prefix and the rest with the carried state (prev_x holds
      the expanded x) equals one shot.
Random vectors have P != R, so a transposed (p, r) index fails (b)-(d).
"""
import numpy as np

import oracle
from synth import custom, make_inputs, make_norm_params

TOL = 1e-12


def _w(rng, H, R, P):
    return rng.uniform(-1.5, 1.5, (H, R, P))


def _case(R, seed=3, T=37):
    w = custom(batch=2, seqlen=T, nheads=3, headdim=5, dstate=8, rank=R, chunk=16, io="f32", seed=seed)
    inp = make_inputs(w)
    rng = np.random.default_rng(seed + 100)
    return w, inp, rng


def _args(inp):
    return inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"], inp["D"]


def _rel(a, b):
    return float(np.abs(np.asarray(a) - np.asarray(b)).max()) / max(float(np.abs(b).max()), 1e-30)


def test_rank1_unit_vectors_is_siso():
    w, inp, rng = _case(1)
    z = rng.standard_normal(inp["x"].shape)
    ones = np.ones((w.nheads, 1, w.headdim))
    y0, f0 = oracle.scan(*_args(inp), z=z)
    y1, f1 = oracle.scan(*_args(inp), z=z, mimo_x=ones, mimo_z=ones, mimo_o=ones)
    assert y1.shape == y0.shape and _rel(y1, y0) < TOL
    for k in f0:
        assert np.allclose(f1[k].reshape(f0[k].shape), f0[k], rtol=0, atol=1e-12), k


def _rank_free(inp, R, rng):
    """x rank-free [B,T,H,P] and the MIMO B, C of rank R from a rank-R workload."""
    x = inp["x"][..., 0].copy()
    return x


def test_expand_x_equals_preexpanded():
    R = 3
    w, inp, rng = _case(R)
    x = _rank_free(inp, R, rng)
    wx = _w(rng, w.nheads, R, w.headdim)
    xe = x[..., None] * np.transpose(wx, (0, 2, 1))[None, None]  # [B,T,H,P,R]
    y_ref, f_ref = oracle.scan(xe, *_args(inp)[1:])
    y, f = oracle.scan(x, *_args(inp)[1:], mimo_x=wx)
    assert y.shape == y_ref.shape and _rel(y, y_ref) < TOL
    for k in f_ref:
        assert _rel(f[k], f_ref[k]) < TOL, k
    # the transposed reading of the vectors gives another result
    wt = np.transpose(wx, (0, 2, 1)).reshape(w.nheads, R, w.headdim)
    y_bad, _ = oracle.scan(x, *_args(inp)[1:], mimo_x=wt)
    assert _rel(y_bad, y_ref) > 1e-3


def test_contract_y_equals_numpy_sum():
    R = 4
    w, inp, rng = _case(R, seed=5)
    wo = _w(rng, w.nheads, R, w.headdim)
    yr, _ = oracle.scan(*_args(inp))                      # [B,T,H,P,R]
    y_ref = np.einsum("bthpr,hrp->bthp", yr, wo)
    y, _ = oracle.scan(*_args(inp), mimo_o=wo)
    assert y.shape == y_ref.shape and _rel(y, y_ref) < TOL


def test_expand_z_equals_preexpanded_gate():
    R = 2
    w, inp, rng = _case(R, seed=7)
    z = rng.standard_normal(inp["x"].shape[:4])
    wz = _w(rng, w.nheads, R, w.headdim)
    ze = z[..., None] * np.transpose(wz, (0, 2, 1))[None, None]
    y_ref, _ = oracle.scan(*_args(inp), z=ze)
    y, _ = oracle.scan(*_args(inp), z=z, mimo_z=wz)
    assert _rel(y, y_ref) < TOL


def test_all_projections_split_schedule():
    R = 3
    w, inp, rng = _case(R, seed=9, T=41)
    x = _rank_free(inp, R, rng)
    z = rng.standard_normal(x.shape)
    wx, wz, wo = (_w(rng, w.nheads, R, w.headdim) for _ in range(3))
    npar = make_norm_params(w)
    kw = dict(mimo_x=wx, mimo_z=wz, mimo_o=wo, **npar)
    rest = _args(inp)[1:]
    y1, f1 = oracle.scan(x, *rest, z=z, **kw)
    # the same composed from numpy: expanded x and z, per-rank outputs contracted
    xe = x[..., None] * np.transpose(wx, (0, 2, 1))[None, None]
    ze = z[..., None] * np.transpose(wz, (0, 2, 1))[None, None]
    yr, fr = oracle.scan(xe, *rest, z=ze, **npar)
    assert _rel(y1, np.einsum("bthpr,hrp->bthp", yr, wo)) < TOL
    assert _rel(f1["prev_x"], fr["prev_x"]) < TOL
    # prefix + rest with the carried state
    t0 = 17
    cut = lambda a, s: a[:, s]
    pre = [cut(a, slice(0, t0)) for a in (x,) + tuple(rest[:5])] + list(rest[5:])
    post = [cut(a, slice(t0, None)) for a in (x,) + tuple(rest[:5])] + list(rest[5:])
    ya, fa = oracle.scan(*pre, z=z[:, :t0], **kw)
    yb, fb = oracle.scan(*post, z=z[:, t0:], init=fa, **kw)
    assert _rel(np.concatenate([ya, yb], axis=1), y1) < 1e-10
    for k in ("h", "prev_B", "prev_x"):
        assert _rel(fb[k], f1[k]) < 1e-10, k
