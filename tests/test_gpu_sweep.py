"""Randomised GPU parity sweep: many small shapes against the fp64 oracle.

Each case draws a shape (batch, heads, T, P, N, rank, chunk, dtype), whether
the norm is on, whether gains/biases and an initial state are given, and
checks y and the carried final state.  Sizes stay small so that the oracle
finishes quickly; every case prints its parameters before touching the GPU.
"""
import numpy as np
import pytest

import oracle
from synth import custom, make_inputs, make_norm_params, make_state
from tests.gpu_util import err_metrics, gate, log, oracle_args, state_to_dev, to_dev, to_np

pytestmark = pytest.mark.gpu


def _cases(n, seed=1234):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 1, 1, 2, 3, 4, 8]))
        Q = int(rng.choice([q for q in (16, 32, 64, 128) if q * R <= 128]))
        N = int(rng.choice([2, 4, 6, 8, 16, 24, 32, 48, 64, 96, 128]))
        P = int(rng.choice([1, 3, 4, 8, 12, 16, 32, 40, 64, 72, 96, 128]))
        T = int(rng.integers(1, 400))
        out.append(dict(batch=int(rng.integers(1, 4)), nheads=int(rng.integers(1, 4)), seqlen=T,
                        headdim=P, dstate=N, rank=R, chunk=Q, io=str(rng.choice(["f32", "bf16"])),
                        bcnorm=bool(rng.random() < 0.8), params=bool(rng.random() < 0.5),
                        init=bool(rng.random() < 0.5), seed=i))
    return out


@pytest.mark.parametrize("case", _cases(40), ids=lambda c: "b{batch}h{nheads}t{seqlen}p{headdim}n{dstate}r{rank}q{chunk}{io}".format(**c))
def test_random_shape(case):
    import torch
    import mamba_selective_scan_amd as m3
    m3.load()
    c = dict(case)
    bcnorm, params, init = c.pop("bcnorm"), c.pop("params"), c.pop("init")
    w = custom(**c)
    log(f"case sweep {w} bcnorm={bcnorm} params={params} init={init}")
    inp = make_inputs(w)
    npar = make_norm_params(w) if params else {}
    st = make_state(w, scale=0.5) if init else None
    y_ref, f_ref = oracle.scan(*oracle_args(inp), bcnorm=bcnorm, init=st, **npar)
    d = to_dev(inp, w.io)
    kw = {k: torch.from_numpy(v).cuda() for k, v in npar.items()}
    if st is not None:
        kw["init"] = state_to_dev(st)
    f = m3.m3_scan_mimo if w.rank > 1 else m3.m3_scan_siso
    y, fin = f(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], chunk=w.chunk,
               bcnorm=bcnorm, final=True, **kw)
    torch.cuda.synchronize()
    raw, comp = err_metrics(to_np(y), y_ref, w.io)
    log(f"  y: raw {raw:.3e} compute {comp:.3e}")
    assert comp <= gate(w.io)
    for k in ("h", "prev_B", "prev_x"):
        r, _ = err_metrics(to_np(fin[k]), f_ref[k], "f32")
        assert r <= (1e-4 if w.io == "f32" else 2e-3), k
