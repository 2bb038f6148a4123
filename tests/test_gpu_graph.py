"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

No entry point allocates, copies, clears memory or synchronises on the stream (the workspace is
the caller's, and every launch is a kernel), so a scan, a run of decode steps or a gradient call
can be captured once and replayed.  Each test replays its graph several times, with eager calls
on other inputs and host synchronisations between the replays, and checks every replay against
the eager result bit for bit (the kernels are deterministic: the same inputs give the same
outputs).
"""
import numpy as np
import pytest

from synth import custom, make_inputs, make_state
from tests.gpu_util import log, state_to_dev, to_dev, to_np

pytestmark = pytest.mark.gpu

FIN = ("h", "prev_B", "prev_x", "angle")


def _m3():
    import mamba_selective_scan_amd as m3
    m3.load()
    return m3


def _same(a, b, what):
    a, b = to_np(a), to_np(b)
    assert a.shape == b.shape, what
    assert np.array_equal(a, b), f"{what}: max |diff| {np.nanmax(np.abs(a - b)):.3e}"


def _scan(m3, d, w, **kw):
    f = m3.m3_scan_mimo if w.rank > 1 else m3.m3_scan_siso
    return f(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], chunk=w.chunk, **kw)


@pytest.mark.parametrize("B,T,H,P,N,R,io,half", [
    (2, 1000, 8, 64, 64, 1, "bf16", False),   # rank-1 16-byte path, folded segments
    (1, 3000, 4, 64, 64, 4, "bf16", False),   # interleaved ranks, the prefix pass
    (1, 2048, 2, 64, 64, 1, "bf16", True),    # half-split pairing in the kernels
    (1, 2048, 2, 64, 32, 1, "bf16", True),    # half-split pairing by permuted copies (N 32)
    (2, 300, 3, 24, 16, 1, "f32", False),     # element path
])
def test_scan_graph_replays(B, T, H, P, N, R, io, half):
    import torch
    m3 = _m3()
    w = custom(batch=B, seqlen=T, nheads=H, headdim=P, dstate=N, rank=R, chunk=64 // R, io=io, seed=T + R)
    log(f"case scan graph {w} half_split={half}")
    inp = make_inputs(w)
    d = to_dev(inp, io)
    init = state_to_dev(make_state(w, scale=0.3))
    kw = dict(half_split=half) if half else {}
    y_e, fin_e = _scan(m3, d, w, init=init, final=True, **kw)
    torch.cuda.synchronize()
    y_g = torch.empty_like(y_e)
    fin_g = m3.new_state(B, H, P, N, R, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _scan(m3, d, w, init=init, final=fin_g, y=y_g, **kw)
    other = to_dev(make_inputs(custom(batch=B, seqlen=T, nheads=H, headdim=P, dstate=N, rank=R, chunk=64 // R,
                                      io=io, seed=T + R + 1)), io)
    for rep in range(3):
        y_g.fill_(float("nan"))
        for k in FIN:
            fin_g[k].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _same(y_g, y_e, f"y, replay {rep}")
        for k in FIN:
            _same(fin_g[k], fin_e[k], f"final {k}, replay {rep}")
        _scan(m3, other, w, final=True, **kw)  # eager work between the replays
        torch.cuda.synchronize()
    log("  3 replays == eager")


def test_decode_steps_graph_replays():
    """Eight decode steps (state updated in place) captured as one graph."""
    import torch
    m3 = _m3()
    w = custom(batch=16, seqlen=8, nheads=4, headdim=64, dstate=64, rank=1, chunk=16, io="bf16", seed=5)
    log(f"case decode graph {w}")
    d = to_dev(make_inputs(w), "bf16")
    st0 = state_to_dev(make_state(w, scale=0.3))
    per_tok = ("x", "B", "C", "dt", "lam", "theta")
    toks = [{k: (v[:, t:t + 1].contiguous() if k in per_tok else v) for k, v in d.items()} for t in range(8)]

    def steps(state, ys):
        for t, o in enumerate(toks):
            m3.m3_step(o["x"], o["B"], o["C"], o["dt"], o["lam"], o["theta"], o["A"], o["D"], state, y=ys[t])

    st_e = {k: v.clone() for k, v in st0.items()}
    ys_e = [torch.empty_like(toks[0]["x"]) for _ in range(8)]
    steps(st_e, ys_e)
    torch.cuda.synchronize()
    st_g = {k: v.clone() for k, v in st0.items()}
    ys_g = [torch.empty_like(toks[0]["x"]) for _ in range(8)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(st_g, ys_g)
    for rep in range(3):
        for k in FIN:
            st_g[k].copy_(st0[k])
        for y in ys_g:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t in range(8):
            _same(ys_g[t], ys_e[t], f"y step {t}, replay {rep}")
        for k in FIN:
            _same(st_g[k], st_e[k], f"state {k}, replay {rep}")
        scratch = {k: v.clone() for k, v in st0.items()}
        steps(scratch, [torch.empty_like(toks[0]["x"]) for _ in range(8)])  # eager work between the replays
        torch.cuda.synchronize()
    log("  3 replays == eager")


def test_gradient_graph_replays():
    """The gradient call (several kernels and a parameter reduction) captured once."""
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=500, nheads=4, headdim=64, dstate=64, rank=1, chunk=64, io="bf16", seed=11)
    log(f"case gradient graph {w}")
    d = to_dev(make_inputs(w), "bf16")
    dy = torch.randn(d["x"].shape, device="cuda").to(torch.bfloat16)
    args = (d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], dy)
    ge = m3.m3_scan_bwd(*args)
    torch.cuda.synchronize()
    ge = {k: v.clone() for k, v in ge.items() if isinstance(v, torch.Tensor)}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gg = m3.m3_scan_bwd(*args)
    gg = {k: v for k, v in gg.items() if isinstance(v, torch.Tensor)}
    assert set(gg) == set(ge) and len(ge) >= 6
    for rep in range(3):
        for v in gg.values():
            v.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k in ge:
            _same(gg[k], ge[k], f"{k}, replay {rep}")
        m3.m3_scan_bwd(*args)  # eager work between the replays
        torch.cuda.synchronize()
    log("  3 replays == eager")
