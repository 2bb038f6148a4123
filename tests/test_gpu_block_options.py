"""GPU parity of the canonical-block options against the fp64 oracle.

Options: partial rotation (rope_pairs), a per-token decay rate A [B, T, H],
softplus(dt + dt_bias) and sigmoid(lambda) input activations and the silu(z)
output gate, on every load path of the scan (rank-1 16-byte path, element
path, interleaved-rank MIMO path, the long-segment prefix path) and on both
decode-step kernels.  Each case prints its name and shape before the GPU runs.
"""
import numpy as np
import pytest

import oracle
from synth import custom, make_block_inputs, make_inputs, make_norm_params, make_state
from tests.gpu_util import angle_err, err_metrics, gate, log, record, state_to_dev, to_np

pytestmark = pytest.mark.gpu

ALL = ("rope", "atok", "softplus", "sigmoid", "gate")


def _m3():
    import mamba_selective_scan_amd as m3
    m3.load()
    return m3


def build_case(w, opts, nr=None):
    """Inputs for the oracle and keyword arguments of the GPU call for a set of options."""
    inp = make_inputs(w)
    ex = make_block_inputs(w, rope_pairs=nr)
    N = w.dstate
    o_kw, g_kw = {}, {}
    theta = inp["theta"]
    if "rope" in opts:
        theta = ex["theta_p"]
        o_kw["rope_pairs"] = g_kw["rope_pairs"] = theta.shape[-1]
    A = ex["A_tok"] if "atok" in opts else inp["A"]
    dt, lam = inp["dt"], inp["lam"]
    if "softplus" in opts:
        dt = ex["dt_raw"]
        o_kw.update(dt_softplus=True, dt_bias=ex["dt_bias"])
        g_kw.update(dt_softplus=True, dt_bias=ex["dt_bias"])
    if "sigmoid" in opts:
        lam = ex["lam_raw"]
        o_kw["lam_sigmoid"] = g_kw["lam_sigmoid"] = True
    if "gate" in opts:
        o_kw["z"] = g_kw["z"] = ex["z"]
    if "half" in opts:
        o_kw["half_split"] = g_kw["half_split"] = True
    data = dict(x=inp["x"], B=inp["B"], C=inp["C"], dt=dt, lam=lam, theta=theta, A=A, D=inp["D"])
    return data, o_kw, g_kw, (theta.shape[-1] if "rope" in opts else N // 2)


def to_gpu(data, g_kw, io):
    import torch
    dev = {}
    for k, v in data.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k in ("x", "B", "C") and io == "bf16":
            t = t.to(torch.bfloat16)
        dev[k] = t.cuda()
    kw = {}
    for k, v in g_kw.items():
        if k == "z":
            t = torch.from_numpy(np.ascontiguousarray(v))
            kw[k] = (t.to(torch.bfloat16) if io == "bf16" else t).cuda()
        elif k == "dt_bias":
            kw[k] = torch.from_numpy(v).cuda()
        else:
            kw[k] = v
    return dev, kw


def check(name, y_gpu, y_ref, io):
    raw, comp = err_metrics(to_np(y_gpu), y_ref, io)
    log(f"  {name}: raw max|err|/rms = {raw:.3e}, compute err = {comp:.3e} (gate {gate(io):.0e})")
    record(name, raw, comp if io == "bf16" else None)
    assert comp <= gate(io), f"{name}: {comp:.3e}"


def check_state(fin_gpu, fin_ref, io):
    for k in ("h", "prev_B", "prev_x"):
        raw, _ = err_metrics(to_np(fin_gpu[k]), fin_ref[k], "f32")
        log(f"  final {k}: max|err|/rms = {raw:.3e}")
        record(f"final {k}", raw)
        assert raw <= (1e-4 if io == "f32" else 2e-3), k
    assert fin_gpu["angle"].shape == fin_ref["angle"].shape
    if fin_ref["angle"].size:
        ae = angle_err(to_np(fin_gpu["angle"]), fin_ref["angle"])
        log(f"  final angle: max wrapped err/rms = {ae:.3e}")
        record("final angle (wrapped)", ae)
        assert ae <= 1e-4


def run_scan(w, opts, *, nr=None, init=True, npar=True):
    import torch
    m3 = _m3()
    log(f"case options {sorted(opts)} nr={nr} {w}")
    data, o_kw, g_kw, NR = build_case(w, opts, nr)
    params = make_norm_params(w) if npar else {}
    st0 = make_state(w, scale=0.4, rope_pairs=NR) if init else None
    y_ref, f_ref = oracle.scan(data["x"], data["B"], data["C"], data["dt"], data["lam"], data["theta"],
                               data["A"], data["D"], init=st0, **params, **o_kw)
    d, kw = to_gpu(data, g_kw, w.io)
    kw.update({k: torch.from_numpy(v).cuda() for k, v in params.items()})
    if st0 is not None:
        kw["init"] = state_to_dev(st0)
    f = m3.m3_scan_mimo if w.rank > 1 else m3.m3_scan_siso
    y, fin = f(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], chunk=w.chunk,
               final=True, **kw)
    torch.cuda.synchronize()
    check("y", y, y_ref, w.io)
    check_state(fin, f_ref, w.io)


# ---------------------------------------------------------------- every option, every load path
@pytest.mark.parametrize("T,P,N,R,Q,io,nr", [
    (300, 64, 64, 1, 64, "bf16", 16),     # rank-1 16-byte path, half the pairs rotate
    (300, 64, 64, 1, 64, "f32", 8),       # rank-1 16-byte path, fp32
    (130, 128, 128, 1, 64, "bf16", 32),   # N 128 with 32 rotated pairs (the 370M layer's rope_fraction)
    (150, 64, 64, 1, 32, "bf16", 6),      # rotated pairs not a multiple of 4: element path
    (77, 5, 6, 1, 16, "f32", 2),          # odd sizes, element path
    (97, 64, 64, 2, 32, "bf16", 8),       # interleaved-rank MIMO path, R 2
    (70, 64, 64, 4, 16, "bf16", 16),      # interleaved-rank MIMO path, R 4
    (40, 32, 16, 3, 16, "f32", 3),        # element path MIMO, R 3
])
def test_all_options(T, P, N, R, Q, io, nr):
    w = custom(batch=2, seqlen=T, nheads=2, headdim=P, dstate=N, rank=R, chunk=Q, io=io, seed=T + nr)
    run_scan(w, set(ALL), nr=nr)


@pytest.mark.parametrize("opt", ALL)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_each_option_alone(opt, io):
    w = custom(batch=2, seqlen=200, nheads=3, headdim=64, dstate=64, chunk=64, io=io, seed=31)
    run_scan(w, {opt}, nr=8 if opt == "rope" else None, init=(opt != "gate"))


@pytest.mark.parametrize("nr", [0, 4, 32])
def test_rope_pairs_extremes(nr):
    """No pair rotates (theta may hold nothing), a few, or all of them through the option."""
    w = custom(batch=2, seqlen=140, nheads=2, headdim=64, dstate=64, chunk=64, io="bf16", seed=41 + nr)
    run_scan(w, {"rope"}, nr=nr)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_all_options_long_segments(io):
    """Many blocks per sequence: sub-segment aggregates and the prefix pass with every option."""
    w = custom(batch=1, seqlen=2048, nheads=2, headdim=32, dstate=32, chunk=16, io=io, seed=77)
    run_scan(w, set(ALL), nr=8)


# ---------------------------------------------------------------- half-split pairing
@pytest.mark.parametrize("T,P,N,R,Q,io,opts", [
    (300, 64, 64, 1, 64, "bf16", ("half",)),                 # rank-1 16-byte path
    (130, 128, 128, 1, 64, "f32", ("half", "rope")),          # N 128, partial rotation
    (77, 5, 6, 1, 16, "f32", ("half",)),                      # odd sizes, element path
    (97, 64, 64, 2, 32, "bf16", ("half",) + ALL),             # MIMO with every option
    (40, 32, 16, 3, 16, "f32", ("half", "gate")),             # element-path MIMO
])
def test_half_split(T, P, N, R, Q, io, opts):
    """Rotation pairs (i, i + N/2): natively on the rank-1 16-byte path with N = 64 or 128
    (rows 1 and 2), on N-permuted copies otherwise; states in and out in the caller's
    (half-split) layout."""
    w = custom(batch=2, seqlen=T, nheads=2, headdim=P, dstate=N, rank=R, chunk=Q, io=io, seed=T + 7)
    run_scan(w, set(opts), nr=N // 4 if "rope" in opts else None)


@pytest.mark.parametrize("T,Q,io,opts", [
    (2048, 16, "bf16", ("half",)),                 # long segments: the prefix pass, permuted copies
    (700, 32, "f32", ("half", "rope", "gate")),    # native pairing over several segments, P 32 tiles
])
def test_half_split_segments(T, Q, io, opts):
    """Half-split pairing over many blocks: the native kernels' carried, folded and final
    states, and the permuted-copy path where the prefix pass runs."""
    w = custom(batch=1, seqlen=T, nheads=2, headdim=32 if io == "f32" else 64, dstate=64, rank=1, chunk=Q, io=io,
               seed=T + Q)
    run_scan(w, set(opts), nr=8 if "rope" in opts else None)


# ---------------------------------------------------------------- decode step and streaming
@pytest.mark.parametrize("R,P,N,io", [(1, 64, 64, "bf16"), (1, 6, 8, "f32"), (2, 16, 32, "f32")])
def test_split_schedule_with_options(R, P, N, io):
    """scan -> steps -> scan with every option and the state in place == one-shot oracle."""
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=150, nheads=2, headdim=P, dstate=N, rank=R, chunk=32, io=io, seed=R + P + N)
    nr = N // 4
    log(f"case split schedule with options nr={nr} {w}")
    data, o_kw, g_kw, NR = build_case(w, set(ALL), nr)
    params = make_norm_params(w)
    st0 = make_state(w, scale=0.3, rope_pairs=NR)
    y_ref, f_ref = oracle.scan(data["x"], data["B"], data["C"], data["dt"], data["lam"], data["theta"],
                               data["A"], data["D"], init=st0, **params, **o_kw)
    d, kw = to_gpu(data, g_kw, io)
    pk = {k: torch.from_numpy(v).cuda() for k, v in params.items()}
    state = state_to_dev(st0)
    scan = m3.m3_scan_mimo if R > 1 else m3.m3_scan_siso
    per_tok = ("x", "B", "C", "dt", "lam", "theta", "A")
    zfull = kw.pop("z")
    pieces, t0 = [], 0
    for kind, n in (("scan", 61), ("step", 3), ("scan", 1), ("step", 1), ("scan", 84)):
        sl = {k: (v[:, t0:t0 + n].contiguous() if k in per_tok else v) for k, v in d.items()}
        zs = zfull[:, t0:t0 + n].contiguous()
        if kind == "scan":
            y, _ = scan(sl["x"], sl["B"], sl["C"], sl["dt"], sl["lam"], sl["theta"], sl["A"], sl["D"],
                        chunk=32, init=state, final=state, z=zs, **kw, **pk)
            pieces.append(y)
        else:
            for k in range(n):
                one = {kk: (vv[:, k:k + 1].contiguous() if kk in per_tok else vv) for kk, vv in sl.items()}
                pieces.append(m3.m3_step(one["x"], one["B"], one["C"], one["dt"], one["lam"], one["theta"],
                                         one["A"], one["D"], state, z=zs[:, k:k + 1].contiguous(), **kw, **pk))
        t0 += n
    assert t0 == w.seqlen
    torch.cuda.synchronize()
    check("y", torch.cat(pieces, dim=1), y_ref, io)
    check_state(state, f_ref, io)


@pytest.mark.parametrize("R,P,N,io", [(1, 64, 64, "bf16"), (2, 16, 32, "f32")])
def test_split_schedule_half_split(R, P, N, io):
    """scan -> steps -> scan with the half-split pairing (the step pairs natively, the scans
    through the permuted copies) == one-shot oracle."""
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=90, nheads=2, headdim=P, dstate=N, rank=R, chunk=32, io=io, seed=R + 11)
    log(f"case split schedule half split {w}")
    data, o_kw, g_kw, NR = build_case(w, {"half"})
    params = make_norm_params(w)
    st0 = make_state(w, scale=0.3)
    y_ref, f_ref = oracle.scan(data["x"], data["B"], data["C"], data["dt"], data["lam"], data["theta"],
                               data["A"], data["D"], init=st0, **params, **o_kw)
    d, kw = to_gpu(data, g_kw, io)
    pk = {k: torch.from_numpy(v).cuda() for k, v in params.items()}
    state = state_to_dev(st0)
    scan = m3.m3_scan_mimo if R > 1 else m3.m3_scan_siso
    per_tok = ("x", "B", "C", "dt", "lam", "theta")  # A is per head here
    pieces, t0 = [], 0
    for kind, n in (("scan", 41), ("step", 2), ("scan", 47)):
        sl = {k: (v[:, t0:t0 + n].contiguous() if k in per_tok else v) for k, v in d.items()}
        if kind == "scan":
            y, _ = scan(sl["x"], sl["B"], sl["C"], sl["dt"], sl["lam"], sl["theta"], sl["A"], sl["D"],
                        chunk=32, init=state, final=state, **kw, **pk)
            pieces.append(y)
        else:
            for k in range(n):
                one = {kk: (vv[:, k:k + 1].contiguous() if kk in per_tok else vv) for kk, vv in sl.items()}
                pieces.append(m3.m3_step(one["x"], one["B"], one["C"], one["dt"], one["lam"], one["theta"],
                                         one["A"], one["D"], state, **kw, **pk))
        t0 += n
    torch.cuda.synchronize()
    check("y", torch.cat(pieces, dim=1), y_ref, io)
    check_state(state, f_ref, io)


@pytest.mark.fullsize
@pytest.mark.parametrize("opts,nr", [(("rope", "atok", "softplus", "sigmoid", "gate"), 16), (("half",), None)])
def test_options_full_workload(opts, nr):
    """The headline workload (batch 4, T 2048, 16 heads, P = N = 64, bf16) with the option sets
    bench.py times: every canonical-block option (16 of 32 pairs rotated), and the half-split
    pairing; y and the final state against the oracle."""
    from synth import WORKLOADS
    run_scan(WORKLOADS[1], set(opts), nr=nr)


def test_option_errors_raise():
    import torch
    m3 = _m3()
    w = custom(batch=1, seqlen=32, nheads=1, headdim=8, dstate=8, io="f32")
    data, _, _, _ = build_case(w, set())
    d, _ = to_gpu(data, {}, "f32")
    log("case option error paths")
    with pytest.raises(RuntimeError, match="M3_EINVAL"):  # more rotated pairs than N/2
        m3.m3_scan_siso(d["x"], d["B"], d["C"], d["dt"], d["lam"], torch.zeros(1, 32, 1, 5, device="cuda"),
                        d["A"], d["D"], chunk=16, rope_pairs=5)
    with pytest.raises(ValueError):  # theta must hold rope_pairs angles
        m3.m3_scan_siso(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], chunk=16,
                        rope_pairs=2)
