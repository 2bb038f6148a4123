"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name, shape and seed before touching the GPU.  Inputs
are the seeded synthetic workloads of ``synth``; the oracle reads the same
(bf16-rounded) values in double precision.
"""
import math

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, custom, make_inputs, make_norm_params, make_state
from tests.gpu_util import (angle_err, err_metrics, gate, head_slice, log, oracle_args, record, state_to_dev,
                            to_dev, to_np)

pytestmark = pytest.mark.gpu


def _m3():
    import mamba_selective_scan_amd as m3
    m3.load()
    return m3


def run_gpu(w, inp, *, chunk=None, init=None, final=False, npar=None, bcnorm=True):
    import torch
    m3 = _m3()
    d = to_dev(inp, w.io)
    kw = dict(chunk=chunk or w.chunk, bcnorm=bcnorm)
    if npar is not None:
        kw.update({k: torch.from_numpy(v).cuda() for k, v in npar.items()})
    if init is not None:
        kw["init"] = state_to_dev(init)
    if final:
        kw["final"] = True
    f = m3.m3_scan_mimo if w.rank > 1 else m3.m3_scan_siso
    out = f(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], **kw)
    torch.cuda.synchronize()
    return out


def check(name, y_gpu, y_ref, io, extra_gate=None):
    raw, comp = err_metrics(to_np(y_gpu), y_ref, io)
    log(f"  {name}: raw max|err|/rms = {raw:.3e}, compute err = {comp:.3e} (gate {gate(io):.0e})")
    record(name, raw, comp if io == "bf16" else None)
    assert comp <= (extra_gate or gate(io)), f"{name}: {comp:.3e}"
    return raw, comp


def check_state(fin_gpu, fin_ref, io):
    for k in ("h", "prev_B", "prev_x"):
        raw, _ = err_metrics(to_np(fin_gpu[k]), fin_ref[k], "f32")
        log(f"  final {k}: max|err|/rms = {raw:.3e}")
        record(f"final {k}", raw)
        assert raw <= (1e-4 if io == "f32" else 2e-3), k
    ae = angle_err(to_np(fin_gpu["angle"]), fin_ref["angle"])
    log(f"  final angle: max wrapped err/rms = {ae:.3e}")
    record("final angle (wrapped)", ae)
    assert ae <= 1e-4


# ---------------------------------------------------------------- the five workloads
@pytest.mark.fullsize
def test_workload0_tiny_fp32():
    w = WORKLOADS[0]
    log(f"case workload0 {w}")
    inp = make_inputs(w)
    y_ref, f_ref = oracle.scan(*oracle_args(inp))
    y, fin = run_gpu(w, inp, final=True)
    check("y", y, y_ref, w.io)
    check_state(fin, f_ref, w.io)


@pytest.mark.fullsize
def test_workload1_siso_bf16():
    w = WORKLOADS[1]
    log(f"case workload1 {w}")
    inp = make_inputs(w)
    y_ref, f_ref = oracle.scan(*oracle_args(inp))
    y, fin = run_gpu(w, inp, final=True)
    check("y", y, y_ref, w.io)
    check_state(fin, f_ref, w.io)


@pytest.mark.fullsize
def test_workload2_mimo_bf16():
    w = WORKLOADS[2]
    log(f"case workload2 {w}")
    inp = make_inputs(w)
    y_ref, f_ref = oracle.scan(*oracle_args(inp))
    y, fin = run_gpu(w, inp, final=True)
    check("y", y, y_ref, w.io)
    check_state(fin, f_ref, w.io)


def test_workload2_mimo_equals_summed_siso_on_gpu():
    """MIMO == R^2 SISO calls (GPU vs GPU), on a slice of the MIMO workload."""
    import torch
    m3 = _m3()
    w = WORKLOADS[2]
    log("case workload2 MIMO vs summed SISO, batch 1, T 512")
    inp = make_inputs(w, batch=1, seqlen=512)
    d = to_dev(inp, w.io)
    y = m3.m3_scan_mimo(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"],
                        chunk=w.chunk)
    zeroD = torch.zeros_like(d["D"])
    ys = torch.zeros(y.shape, dtype=torch.float32, device="cuda")
    for r in range(w.rank):
        for rp in range(w.rank):
            ys[..., r] += m3.m3_scan_siso(d["x"][..., rp].contiguous(), d["B"][..., rp].contiguous(),
                                          d["C"][..., r].contiguous(), d["dt"], d["lam"], d["theta"],
                                          d["A"], zeroD, chunk=64).float()
        ys[..., r] += d["D"][None, None, :, None] * d["x"][..., r].float()
    y_ref, _ = oracle.scan(*oracle_args(inp))
    check("mimo", y, y_ref, w.io)
    # the summed SISO outputs went through R^2 bf16 roundings: allow R^2 output quanta
    raw, comp = err_metrics(to_np(ys), y_ref, "bf16")
    log(f"  summed siso: raw {raw:.3e}")
    assert raw <= 4 * w.rank * w.rank * 2.0 ** -8 * np.abs(y_ref).max() / math.sqrt(np.mean(y_ref ** 2))


@pytest.mark.fullsize
def test_workload3_long_bf16():
    w = WORKLOADS[3]
    log(f"case workload3 {w}")
    inp = make_inputs(w)
    y_ref, f_ref = oracle.scan(*oracle_args(inp))
    y, fin = run_gpu(w, inp, final=True)
    check("y", y, y_ref, w.io)
    check_state(fin, f_ref, w.io)


@pytest.mark.fullsize
def test_workload4_decode_512_steps():
    """512 consecutive m3_step calls vs the oracle's full scan over the same tokens."""
    import torch
    m3 = _m3()
    w = WORKLOADS[4]
    log(f"case workload4 {w}")
    inp = make_inputs(w)
    d = to_dev(inp, w.io)
    Bsz, T, H = inp["dt"].shape
    # token-major copies so each step reads contiguous [B, 1, H, ...] slices
    tm = {k: (v.transpose(0, 1).contiguous() if k not in ("A", "D") else v) for k, v in d.items()}
    state = m3.new_state(Bsz, H, w.headdim, w.dstate, 1)
    ys = torch.empty_like(d["x"])
    for t in range(T):
        yt = m3.m3_step(tm["x"][t].unsqueeze(1), tm["B"][t].unsqueeze(1), tm["C"][t].unsqueeze(1),
                        tm["dt"][t].unsqueeze(1), tm["lam"][t].unsqueeze(1), tm["theta"][t].unsqueeze(1),
                        d["A"], d["D"], state)
        ys[:, t:t + 1] = yt
    torch.cuda.synchronize()
    # every batch row: y of all 512 tokens and the carried state after them
    y_ref, f_ref = oracle.scan(*oracle_args(inp))
    check("y (all 256 batch rows x 512 steps)", ys, y_ref, w.io)
    check_state(state, f_ref, w.io)


# ---------------------------------------------------------------- chunk size invariance
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_chunk_size_invariance(io):
    """Blocks of 16, 32 and 64 tokens give the oracle's result.  A requested chunk of 128 is
    accepted and runs as 64-token blocks (the block height is 64 rows): bit for bit the
    result of chunk 64."""
    w = custom(batch=2, seqlen=300, nheads=3, headdim=64, dstate=64, io=io, seed=7)
    log(f"case chunk invariance {w}")
    inp = make_inputs(w)
    y_ref, f_ref = oracle.scan(*oracle_args(inp))
    out = {}
    for Q in (16, 32, 64, 128):
        y, fin = run_gpu(w, inp, chunk=Q, final=True)
        check(f"Q={Q}", y, y_ref, io)
        check_state(fin, f_ref, io)
        out[Q] = (to_np(y), {k: to_np(v) for k, v in fin.items()})
    assert np.array_equal(out[128][0], out[64][0])
    for k in out[64][1]:
        assert np.array_equal(out[128][1][k], out[64][1][k]), k


# ---------------------------------------------------------------- shapes and edge cases
@pytest.mark.parametrize("T,P,N,R,Q,io", [
    (1, 64, 64, 1, 64, "bf16"),        # one token
    (65, 64, 64, 1, 64, "bf16"),       # ragged tail of one token
    (200, 16, 32, 1, 32, "f32"),       # small P, N
    (77, 3, 6, 1, 16, "f32"),          # N, P not multiples of 8
    (50, 1, 2, 1, 16, "f32"),          # smallest sizes
    (130, 128, 128, 1, 64, "bf16"),    # largest P and N
    (97, 64, 64, 2, 32, "bf16"),       # MIMO R=2, ragged
    (70, 64, 64, 4, 16, "bf16"),       # MIMO R=4 (16-byte interleaved-rank loads), ragged
    (45, 40, 48, 8, 16, "bf16"),       # MIMO R=8, N and P not powers of two
    (60, 128, 128, 4, 16, "bf16"),     # MIMO R=4 at the largest N and P
    (40, 32, 16, 3, 16, "f32"),        # MIMO R=3 (48 rows -> 64 padded)
    (33, 16, 32, 8, 16, "f32"),        # MIMO R=8, 128 rows
])
def test_shapes(T, P, N, R, Q, io):
    w = custom(batch=2, seqlen=T, nheads=2, headdim=P, dstate=N, rank=R, chunk=Q, io=io, seed=T + P + N)
    log(f"case shapes {w}")
    inp = make_inputs(w)
    inp["dt"] = (inp["dt"] * 3).astype(np.float32)
    npar = make_norm_params(w)
    y_ref, f_ref = oracle.scan(*oracle_args(inp), **npar)
    y, fin = run_gpu(w, inp, final=True, npar=npar)
    check("y", y, y_ref, io)
    check_state(fin, f_ref, io)


@pytest.mark.parametrize("io,with_params", [("f32", False), ("bf16", False), ("f32", True), ("bf16", True)])
def test_norm_off_and_nonzero_init(io, with_params):
    """Norm off (gains then have no effect, biases still apply) with a carried initial state."""
    w = custom(batch=2, seqlen=150, nheads=2, headdim=32, dstate=32, chunk=32, io=io, seed=99)
    log(f"case norm off + init {w} params={with_params}")
    inp = make_inputs(w)
    st = make_state(w, scale=0.5)
    npar = make_norm_params(w) if with_params else {}
    y_ref, f_ref = oracle.scan(*oracle_args(inp), bcnorm=False, init=st, **npar)
    y, fin = run_gpu(w, inp, init=st, final=True, bcnorm=False, npar=npar or None)
    check("y", y, y_ref, io)
    check_state(fin, f_ref, io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_long_segments_with_state(io):
    """Few sequences and many blocks: the state is aggregated over sub-segments shorter than
    the output segments and a prefix pass assembles every segment's incoming state,
    including the initial state."""
    w = custom(batch=1, seqlen=2048, nheads=2, headdim=32, dstate=32, chunk=16, io=io, seed=2048)
    log(f"case long segments + init {w}")
    inp = make_inputs(w)
    st = make_state(w, scale=0.5)
    npar = make_norm_params(w)
    y_ref, f_ref = oracle.scan(*oracle_args(inp), init=st, **npar)
    y, fin = run_gpu(w, inp, init=st, final=True, npar=npar)
    check("y", y, y_ref, io)
    check_state(fin, f_ref, io)


def test_empty_sequence_copies_state():
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=0, nheads=2, headdim=8, dstate=8, io="f32", seed=1)
    log(f"case empty {w}")
    inp = make_inputs(w)
    st = make_state(w)
    d = to_dev(inp, "f32")
    y, fin = m3.m3_scan_siso(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"],
                             chunk=16, init=state_to_dev(st), final=True)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 2, 8)
    for k in ("h", "prev_B", "prev_x"):
        assert np.array_equal(to_np(fin[k]), st[k].astype(np.float64))
    assert angle_err(to_np(fin["angle"]), st["angle"]) < 1e-6


def test_reduces_to_mamba2_on_gpu():
    """lambda = 1, theta = 0: the Mamba-2 recurrence (oracle pin P2 reduction) on the GPU."""
    from tests import pinforms as pf
    w = custom(batch=2, seqlen=256, nheads=2, headdim=32, dstate=32, chunk=64, io="f32", seed=5)
    log(f"case mamba2 reduction {w}")
    inp = make_inputs(w)
    inp["lam"] = np.ones_like(inp["lam"])
    inp["theta"] = np.zeros_like(inp["theta"])
    y2 = pf.mamba2_loop(inp["x"], inp["B"], inp["C"], inp["dt"], inp["A"], inp["D"], bcnorm=True)
    y = run_gpu(w, inp)
    check("mamba2", y, y2, "f32")


def test_closed_form_on_gpu():
    from tests import pinforms as pf
    T, N, dt, A, lam, th = 300, 8, 0.3, -0.7, 0.35, 0.2
    log("case closed form on gpu")
    w = custom(batch=1, seqlen=T, nheads=1, headdim=1, dstate=N, chunk=64, io="f32")
    inp = dict(x=np.ones((1, T, 1, 1), np.float32), B=np.ones((1, T, 1, N), np.float32),
               C=np.ones((1, T, 1, N), np.float32), dt=np.full((1, T, 1), dt, np.float32),
               lam=np.full((1, T, 1), lam, np.float32), theta=np.full((1, T, 1, N // 2), th, np.float32),
               A=np.array([A], np.float32), D=np.zeros(1, np.float32))
    y = run_gpu(w, inp, bcnorm=False)
    ref = pf.closed_form(T, N, float(np.float32(dt)), float(np.float32(A)), float(np.float32(lam)),
                         float(np.float32(th)))
    check("closed form", y[0, :, 0, 0], ref, "f32")


# ---------------------------------------------------------------- streaming
@pytest.mark.parametrize("io,R", [("f32", 1), ("bf16", 1), ("f32", 2)])
def test_split_schedule_scan_step_scan(io, R):
    """scan(prefix) -> m3_step x k -> scan(rest) with the state in place == one-shot."""
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=203, nheads=2, headdim=32, dstate=32, rank=R, chunk=32, io=io, seed=13)
    log(f"case split schedule {w}")
    inp = make_inputs(w)
    st0 = make_state(w, scale=0.3)
    y_ref, f_ref = oracle.scan(*oracle_args(inp), init=st0)
    d = to_dev(inp, io)
    state = state_to_dev(st0)
    scan = m3.m3_scan_mimo if R > 1 else m3.m3_scan_siso
    pieces, t0 = [], 0
    for kind, n in (("scan", 70), ("step", 3), ("scan", 1), ("step", 1), ("scan", 128)):
        sl = {k: (v[:, t0:t0 + n].contiguous() if k not in ("A", "D") else v) for k, v in d.items()}
        if kind == "scan":
            y, _ = scan(sl["x"], sl["B"], sl["C"], sl["dt"], sl["lam"], sl["theta"], sl["A"], sl["D"],
                        chunk=32, init=state, final=state)
            pieces.append(y)
        else:
            for k in range(n):
                one = {kk: (vv[:, k:k + 1].contiguous() if kk not in ("A", "D") else vv) for kk, vv in sl.items()}
                pieces.append(m3.m3_step(one["x"], one["B"], one["C"], one["dt"], one["lam"], one["theta"],
                                         one["A"], one["D"], state))
        t0 += n
    assert t0 == w.seqlen
    torch.cuda.synchronize()
    check("y", torch.cat(pieces, dim=1), y_ref, io)
    check_state(state, f_ref, io)


def test_step_matches_scan_mimo_f32():
    import torch
    m3 = _m3()
    w = custom(batch=3, seqlen=20, nheads=2, headdim=8, dstate=16, rank=4, chunk=16, io="f32", seed=17)
    log(f"case step mimo {w}")
    inp = make_inputs(w)
    npar = make_norm_params(w)
    y_ref, f_ref = oracle.scan(*oracle_args(inp), **npar)
    d = to_dev(inp, "f32")
    pd = {k: torch.from_numpy(v).cuda() for k, v in npar.items()}
    state = m3.new_state(3, 2, 8, 16, 4)
    ys = []
    for t in range(w.seqlen):
        one = {k: (v[:, t:t + 1].contiguous() if k not in ("A", "D") else v) for k, v in d.items()}
        ys.append(m3.m3_step(one["x"], one["B"], one["C"], one["dt"], one["lam"], one["theta"],
                             one["A"], one["D"], state, **pd))
    torch.cuda.synchronize()
    check("y", torch.cat(ys, 1), y_ref, "f32")
    check_state(state, f_ref, "f32")


@pytest.mark.parametrize("N,P,io", [(6, 12, "f32"), (6, 5, "f32"), (128, 128, "bf16"), (64, 64, "bf16")])
def test_step_rank1_shapes(N, P, io):
    """Rank-1 steps (norm gains and biases, initial state) vs the oracle's scan over the same
    tokens: odd pair counts, P not a multiple of 4 (element path), the largest N and P."""
    import torch
    m3 = _m3()
    w = custom(batch=3, seqlen=12, nheads=2, headdim=P, dstate=N, chunk=16, io=io, seed=N + P)
    log(f"case step rank 1 {w}")
    inp = make_inputs(w)
    npar = make_norm_params(w)
    st0 = make_state(w, scale=0.4)
    y_ref, f_ref = oracle.scan(*oracle_args(inp), init=st0, **npar)
    d = to_dev(inp, io)
    pd = {k: torch.from_numpy(v).cuda() for k, v in npar.items()}
    state = state_to_dev(st0)
    ys = []
    for t in range(w.seqlen):
        one = {k: (v[:, t:t + 1].contiguous() if k not in ("A", "D") else v) for k, v in d.items()}
        ys.append(m3.m3_step(one["x"], one["B"], one["C"], one["dt"], one["lam"], one["theta"],
                             one["A"], one["D"], state, **pd))
    torch.cuda.synchronize()
    check("y", torch.cat(ys, 1), y_ref, io)
    check_state(state, f_ref, io)


def test_errors_raise():
    import torch
    m3 = _m3()
    w = custom(batch=1, seqlen=32, nheads=1, headdim=8, dstate=8, io="f32")
    d = to_dev(make_inputs(w), "f32")
    log("case error paths on device tensors")
    with pytest.raises(RuntimeError, match="M3_EUNSUPPORTED"):
        m3.m3_scan_siso(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], chunk=48)
    with pytest.raises(RuntimeError, match="M3_EWORKSPACE"):
        m3.m3_scan_siso(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], chunk=16,
                        workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))


def test_side_stream_scan_and_gradients():
    """Scan and gradient calls issued on a non-current stream (outputs and workspace then
    belong to that stream) match the same calls on the current stream, with other work
    queued on the current stream meanwhile."""
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=600, nheads=4, headdim=64, dstate=64, io="bf16", seed=31)
    log(f"case side stream {w}")
    inp = make_inputs(w)
    d = to_dev(inp, w.io)
    args = (d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"])
    y0, f0 = m3.m3_scan_siso(*args, chunk=64, final=True)
    dy = torch.randn_like(y0.float()).to(y0.dtype)
    g0 = m3.m3_scan_bwd(*args, dy)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        y1, f1 = m3.m3_scan_siso(*args, chunk=64, final=True, stream=side)
        g1 = m3.m3_scan_bwd(*args, dy, stream=side)
        # allocations on the current stream while the side stream still runs
        junk = [torch.empty(1 << 22, dtype=torch.uint8, device="cuda").fill_(7) for _ in range(4)]
        outs.append((y1, f1, g1))
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for y1, f1, g1 in outs:
        assert torch.equal(y1, y0)
        for k in f0:
            assert torch.equal(f1[k], f0[k]), k
        for k in ("x", "B", "C", "dt", "lam", "theta", "A", "D"):
            assert torch.equal(g1[k], g0[k]), k
