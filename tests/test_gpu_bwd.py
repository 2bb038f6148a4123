"""GPU parity of the scan's gradients (m3_scan_bwd) against the fp64 oracle's reverse sweep.

The oracle's gradients are pinned by finite differences (tests/test_oracle_bwd_pins.py).
Each case prints its name and shape before the GPU runs.

Gates (max |err| / max(rms of the oracle gradient, 1e-3)): 2e-4 for every gradient computed in
float32 (the sweeps accumulate over T tokens in fp32); gradients stored in bf16 (dx, dB,
dC, dz of bf16 calls) are first allowed their own rounding, 2^-8 |g|, as y is.
"""
import math

import numpy as np
import pytest

import oracle
from synth import custom, make_block_inputs, make_inputs, make_norm_params, make_state
from tests.gpu_util import log, record

pytestmark = pytest.mark.gpu

GATE = 2e-4
HALF_ULP = 2.0 ** -8


def _m3():
    import mamba_selective_scan_amd as m3
    m3.load()
    return m3


def _err(g, ref, io_rounded):
    g = np.asarray(g, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    # a gradient that is exactly zero in exact arithmetic (e.g. of the initial angle with a
    # zero initial state and no final-state gradient) is compared against a floor of 1e-3,
    # three orders below the gradients of these O(1) inputs
    rms = max(math.sqrt(float(np.mean(ref * ref))), 1e-3)
    d = np.abs(g - ref)
    if io_rounded:
        d = np.maximum(d - HALF_ULP * np.abs(ref), 0.0)
    return float(d.max()) / rms


def run_case(w, *, opts=(), nr=None, init=True, dfinal=True, npar=True, bcnorm=True):
    import torch
    m3 = _m3()
    log(f"case bwd opts={sorted(opts)} nr={nr} init={init} dfinal={dfinal} norm={bcnorm} {w}")
    inp = make_inputs(w)
    ex = make_block_inputs(w, rope_pairs=nr)
    data = dict(x=inp["x"], B=inp["B"], C=inp["C"], dt=inp["dt"] * 4, lam=inp["lam"], theta=inp["theta"],
                A=inp["A"], D=inp["D"])
    kw = {}
    NR = w.dstate // 2
    if "rope" in opts:
        data["theta"] = ex["theta_p"]
        kw["rope_pairs"] = NR = ex["theta_p"].shape[-1]
    if "atok" in opts:
        data["A"] = ex["A_tok"]
    if "act" in opts:
        data["dt"], data["lam"] = ex["dt_raw"], ex["lam_raw"]
        kw.update(dt_softplus=True, dt_bias=ex["dt_bias"], lam_sigmoid=True)
    if "gate" in opts:
        kw["z"] = ex["z"]
    if "half" in opts:
        kw["half_split"] = True
    params = make_norm_params(w) if npar else {}
    st0 = make_state(w, scale=0.4, rope_pairs=NR) if init else None
    rng = np.random.default_rng(w.seed + 5)
    dy = rng.standard_normal(np.shape(data["x"])).astype(np.float32)
    if w.io == "bf16":
        from synth import bf16_round
        dy = bf16_round(dy)
    dfin = None
    if dfinal:
        R = w.rank
        dfin = dict(h=rng.standard_normal((w.batch, w.nheads, w.dstate, w.headdim)).astype(np.float32),
                    prev_B=rng.standard_normal((w.batch, w.nheads, w.dstate, R)).astype(np.float32),
                    prev_x=rng.standard_normal((w.batch, w.nheads, w.headdim, R)).astype(np.float32),
                    angle=rng.standard_normal((w.batch, w.nheads, NR)).astype(np.float32))
    ref = oracle.scan_bwd(*data.values(), dy, bcnorm=bcnorm, init=st0, dfinal=dfin, **params, **kw)
    # device tensors
    bf = torch.bfloat16 if w.io == "bf16" else torch.float32
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in data.items()}
    for k in ("x", "B", "C"):
        dev[k] = dev[k].to(bf)
    gk = {k: (torch.from_numpy(v).cuda() if isinstance(v, np.ndarray) else v) for k, v in kw.items()}
    if "z" in gk:
        gk["z"] = gk["z"].to(bf)
    gk.update({k: torch.from_numpy(v).cuda() for k, v in params.items()})
    sd = lambda st: {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda() for k, v in st.items()}
    g = m3.m3_scan_bwd(*dev.values(), torch.from_numpy(dy).cuda().to(bf), bcnorm=bcnorm,
                       init=sd(st0) if st0 is not None else None, dfinal=sd(dfin) if dfin is not None else None,
                       **gk)
    torch.cuda.synchronize()
    bad = []
    names = ["x", "B", "C", "dt", "lam", "theta", "A", "D", "b_bias", "c_bias"]
    if bcnorm:
        names += ["b_norm_w", "c_norm_w"]
    if "act" in opts:
        names.append("dt_bias")
    if "gate" in opts:
        names.append("z")
    for k in names:
        got = g[k].float().cpu().numpy()
        e = _err(got, ref[k], w.io == "bf16" and k in ("x", "B", "C", "z"))
        log(f"  d{k}: {e:.3e}")
        record(f"d{k}", e)
        if not e <= GATE:
            bad.append((k, e))
    for k in ("h", "prev_B", "prev_x", "angle"):
        e = _err(g["init"][k].cpu().numpy(), ref["init"][k], False)
        log(f"  dinit.{k}: {e:.3e}")
        record(f"dinit.{k}", e)
        if not e <= GATE:
            bad.append(("init." + k, e))
    assert not bad, bad


def test_bwd_tiny_f32():
    run_case(custom(batch=1, seqlen=40, nheads=2, headdim=8, dstate=8, io="f32", seed=1))


@pytest.mark.parametrize("T,P,N,R,io", [
    (100, 64, 64, 1, "f32"),     # several 16-token blocks and a ragged tail
    (100, 64, 64, 1, "bf16"),
    (77, 5, 6, 1, "f32"),        # odd sizes, odd pair count
    (130, 128, 128, 1, "f32"),   # largest N and P
    (50, 16, 32, 2, "f32"),      # MIMO R 2
    (41, 8, 16, 3, "f32"),       # MIMO R 3 (5 tokens per block)
    (30, 64, 64, 4, "bf16"),     # MIMO R 4
    (1, 16, 16, 1, "f32"),       # a single token (the last token is the first)
    (64, 32, 32, 1, "bf16"),     # exactly one chunk
    (129, 32, 64, 1, "f32"),     # one token past two chunks
    (33, 16, 16, 8, "f32"),      # MIMO R 8 (8 tokens per chunk)
    (70, 128, 32, 1, "bf16"),    # P 128 with N 32
    (45, 24, 40, 5, "f32"),      # MIMO R 5, N and P not multiples of 16
    (90, 128, 64, 1, "f32"),     # chunk states staged one side at a time (P 128)
    (75, 48, 128, 2, "f32"),     # the same with N 128, MIMO R 2
])
def test_bwd_shapes(T, P, N, R, io):
    run_case(custom(batch=2, seqlen=T, nheads=2, headdim=P, dstate=N, rank=R, io=io, seed=T + N + R))


@pytest.mark.parametrize("R", [1, 2])
def test_bwd_all_options(R):
    w = custom(batch=2, seqlen=90, nheads=2, headdim=32, dstate=32, rank=R, io="f32", seed=17 + R)
    run_case(w, opts=("rope", "atok", "act", "gate"), nr=8)


@pytest.mark.parametrize("R,N,P,io,opts", [
    (1, 32, 32, "bf16", ("half",)),                                 # N 32: N-permuted copies
    (2, 32, 32, "f32", ("half", "rope", "atok", "act", "gate")),    # N 32: N-permuted copies
    (1, 64, 32, "bf16", ("half",)),                                 # N 64: pairs in the kernels
    (2, 64, 48, "f32", ("half", "rope", "atok", "act", "gate")),    # N 64, rank 2, every option
    (1, 128, 64, "bf16", ("half", "rope")),                         # N 128, partial rotation
    (3, 128, 24, "f32", ("half",)),                                 # N 128, rank 3 (element loads)
])
def test_bwd_half_split(R, N, P, io, opts):
    """Gradients with the half-split pairing: paired in the kernels at N = 64 or 128, through
    N-permuted copies in the workspace otherwise."""
    w = custom(batch=2, seqlen=90, nheads=2, headdim=P, dstate=N, rank=R, io=io, seed=29 + R + N)
    run_case(w, opts=opts, nr=(N // 4 if N >= 64 else 8) if "rope" in opts else None)


def test_bwd_norm_off_no_state():
    w = custom(batch=2, seqlen=64, nheads=3, headdim=16, dstate=16, io="f32", seed=23)
    run_case(w, init=False, dfinal=False, bcnorm=False)


def test_bwd_empty_sequence():
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=0, nheads=2, headdim=8, dstate=8, io="f32", seed=2)
    log(f"case bwd empty {w}")
    inp = make_inputs(w)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    st0 = make_state(w)
    rng = np.random.default_rng(0)
    dfin = dict(h=rng.standard_normal((2, 2, 8, 8)), prev_B=rng.standard_normal((2, 2, 8, 1)),
                prev_x=rng.standard_normal((2, 2, 8, 1)), angle=rng.standard_normal((2, 2, 4)))
    sd = lambda st: {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda() for k, v in st.items()}
    g = m3.m3_scan_bwd(dev["x"], dev["B"], dev["C"], dev["dt"], dev["lam"], dev["theta"], dev["A"], dev["D"],
                       torch.zeros_like(dev["x"]), init=sd(st0), dfinal=sd(dfin))
    torch.cuda.synchronize()
    for k in ("h", "prev_B", "prev_x", "angle"):
        assert np.array_equal(g["init"][k].cpu().numpy(), dfin[k].astype(np.float32))
    assert float(g["D"].abs().sum()) == 0.0 and float(g["A"].abs().sum()) == 0.0


@pytest.mark.parametrize("with_init", [False, True])
def test_bwd_without_initial_state_gradients(with_init):
    """dinit = NULL (init_grad=False) leaves every other gradient bit-identical; without an
    initial state the initial-state kernel is skipped and its eta term taken as zero."""
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=150, nheads=3, headdim=32, dstate=32, io="bf16", seed=31)
    log(f"case bwd init_grad=False with_init={with_init} {w}")
    inp = make_inputs(w)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    for k in ("x", "B", "C"):
        dev[k] = dev[k].to(torch.bfloat16)
    kw = {}
    if with_init:
        kw["init"] = {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda()
                      for k, v in make_state(w, scale=0.5).items()}
    dy = torch.randn(dev["x"].shape, device="cuda").to(torch.bfloat16)
    args = (dev["x"], dev["B"], dev["C"], dev["dt"], dev["lam"], dev["theta"], dev["A"], dev["D"], dy)
    ga = m3.m3_scan_bwd(*args, **kw)
    gb = m3.m3_scan_bwd(*args, init_grad=False, **kw)
    torch.cuda.synchronize()
    assert gb["init"] is None
    for k, v in ga.items():
        if isinstance(v, torch.Tensor):
            assert torch.equal(v, gb[k]), k


@pytest.mark.fullsize
@pytest.mark.parametrize("opts", [("rope", "atok", "act", "gate"), ("half",)])
def test_bwd_full_workload_options(opts):
    """Gradients at the headline workload's full size with every canonical-block option (16 of
    32 pairs rotated) and with the half-split pairing, against the oracle's reverse sweep."""
    from synth import WORKLOADS
    run_case(WORKLOADS[1], opts=opts, nr=16 if "rope" in opts else None)


@pytest.mark.fullsize
@pytest.mark.parametrize("k", [1, 2, 3])
def test_bwd_full_workloads(k):
    """The bench workloads at full size (SISO config, MIMO rank 4, the 16384-token N 128 one):
    every gradient against the oracle's reverse sweep on the same inputs, with norm gains and
    biases, an initial state and final-state gradients."""
    import torch
    from synth import WORKLOADS, bf16_round
    m3 = _m3()
    w = WORKLOADS[k]
    log(f"case bwd full workload {k} {w}")
    inp = make_inputs(w)
    params = make_norm_params(w)
    st0 = make_state(w, scale=0.4)
    rng = np.random.default_rng(w.seed + 5)
    dy = bf16_round(rng.standard_normal(np.shape(inp["x"])).astype(np.float32))
    R, NR = w.rank, w.dstate // 2
    dfin = dict(h=rng.standard_normal((w.batch, w.nheads, w.dstate, w.headdim)).astype(np.float32),
                prev_B=rng.standard_normal((w.batch, w.nheads, w.dstate, R)).astype(np.float32),
                prev_x=rng.standard_normal((w.batch, w.nheads, w.headdim, R)).astype(np.float32),
                angle=rng.standard_normal((w.batch, w.nheads, NR)).astype(np.float32))
    data = [inp[n] for n in ("x", "B", "C", "dt", "lam", "theta", "A", "D")]
    ref = oracle.scan_bwd(*data, dy, init=st0, dfinal=dfin, **params)
    bf = torch.bfloat16 if w.io == "bf16" else torch.float32
    dev = [torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in data]
    for i in range(3):
        dev[i] = dev[i].to(bf)
    sd = lambda st: {kk: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda() for kk, v in st.items()}
    g = m3.m3_scan_bwd(*dev, torch.from_numpy(dy).cuda().to(bf), init=sd(st0), dfinal=sd(dfin),
                       **{kk: torch.from_numpy(v).cuda() for kk, v in params.items()})
    torch.cuda.synchronize()
    bad = []
    for name in ("x", "B", "C", "dt", "lam", "theta", "A", "D", "b_bias", "c_bias", "b_norm_w", "c_norm_w"):
        e = _err(g[name].float().cpu().numpy(), ref[name], w.io == "bf16" and name in ("x", "B", "C"))
        log(f"  d{name}: {e:.3e}")
        record(f"d{name}", e)
        if not e <= GATE:
            bad.append((name, e))
    for name in ("h", "prev_B", "prev_x", "angle"):
        e = _err(g["init"][name].cpu().numpy(), ref["init"][name], False)
        log(f"  dinit.{name}: {e:.3e}")
        record(f"dinit.{name}", e)
        if not e <= GATE:
            bad.append(("init." + name, e))
    assert not bad, bad
