"""GPU parity of the MIMO projections by learned per-rank vectors (mimo_x, mimo_z,
mimo_o) and of row-strided inputs (slices of a wider in_proj-like buffer).

torchmamba README, "Math notes", MIMO paragraph (per-head x / z expanded and y
contracted by learned vectors); dotLLM PR #136, "What's deferred" (MIMO-in-Block:
the mimo_x / mimo_z projections and the post-scan rank contraction) and "Stage C"
(in_proj GEMM, then the split into the scan's inputs).

Every case prints its name and shape before the GPU runs.  The fp64 oracle takes
the projections itself, except for mimo_x on bf16 I/O: the library forms
x_r = x * mimo_x[h, r] in fp32 and rounds it once to bf16 (as an unexpanded bf16 x
arrives), so there the oracle reads that rounded x_r, formed here with numpy (one
fp32 product and one round-to-nearest-even per element, the library's documented
rounding), and the carried prev_x must hold exactly those values.
"""
import numpy as np
import pytest

import oracle
from synth import bf16_round, custom, make_block_inputs, make_inputs, make_mimo_proj, make_norm_params, make_state
from tests.gpu_util import angle_err, err_metrics, gate, log, record, state_to_dev, to_np

pytestmark = pytest.mark.gpu


def _m3():
    import mamba_selective_scan_amd as m3
    m3.load()
    return m3


def _dev(a, io, big=False):
    """numpy -> device tensor; x-like arrays (big) in the io dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if big and io == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def expand_x_bf16(x_free, mimo_x):
    """x_r[b, t, h, p, r] = bf16(fp32(x[b, t, h, p] * mimo_x[h, r, p]))."""
    prod = (x_free[..., None].astype(np.float32) * np.transpose(mimo_x, (0, 2, 1))[None, None].astype(np.float32))
    return bf16_round(prod.astype(np.float32))


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
    if fin_ref["angle"].size:
        ae = angle_err(to_np(fin_gpu["angle"]), fin_ref["angle"])
        log(f"  final angle: max wrapped err/rms = {ae:.3e}")
        record("final angle (wrapped)", ae)
        assert ae <= 1e-4


def proj_case(w, which, *, gate_z=True, init=True):
    """Oracle inputs / keyword arguments and GPU arguments of one projection case."""
    inp = make_inputs(w)
    pj = make_mimo_proj(w)
    ex = make_block_inputs(w)
    params = make_norm_params(w)
    o_kw = dict(params)
    g = dict(x=inp["x"], B=inp["B"], C=inp["C"], dt=inp["dt"], lam=inp["lam"], theta=inp["theta"],
             A=inp["A"], D=inp["D"])
    ox = inp["x"]
    if "x" in which:
        g["x"] = pj["x_free"]
        g["mimo_x"] = pj["mimo_x"]
        if w.io == "bf16":
            ox = expand_x_bf16(pj["x_free"], pj["mimo_x"])
        else:
            ox = pj["x_free"]
            o_kw["mimo_x"] = pj["mimo_x"]
    if gate_z:
        if "z" in which:
            g["z"] = o_kw["z"] = pj["z_free"]
            g["mimo_z"] = o_kw["mimo_z"] = pj["mimo_z"]
        else:
            g["z"] = o_kw["z"] = ex["z"]
    if "o" in which:
        g["mimo_o"] = o_kw["mimo_o"] = pj["mimo_o"]
    st0 = make_state(w, scale=0.4) if init else None
    return inp, ox, o_kw, g, params, st0


def gpu_kwargs(g, params, w):
    """Device arguments; at rank 1 the MIMO entry points take B, C (and a rank-full x, z) with
    a trailing rank axis of 1."""
    kw = {}
    for k, v in g.items():
        if k in ("x", "B", "C", "z"):
            full = k in ("B", "C") or (k == "x" and "mimo_x" not in g) or (k == "z" and "mimo_z" not in g)
            if w.rank == 1 and full:
                v = v[..., None]
            kw[k] = _dev(v, w.io, big=True)
        else:
            kw[k] = _dev(v, w.io)
    kw.update({k: _dev(v, w.io) for k, v in params.items()})
    return kw


def run_proj(w, which, **kw):
    import torch
    m3 = _m3()
    log(f"case projections {sorted(which)} {w}")
    inp, ox, o_kw, g, params, st0 = proj_case(w, which, **kw)
    y_ref, f_ref = oracle.scan(ox, inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"], inp["D"],
                               init=st0, **o_kw)
    d = gpu_kwargs(g, params, w)
    args = [d.pop(k) for k in ("x", "B", "C", "dt", "lam", "theta", "A", "D")]
    if st0 is not None:
        d["init"] = state_to_dev(st0)
    y, fin = m3.m3_scan_mimo(*args, chunk=w.chunk, final=True, **d)
    torch.cuda.synchronize()
    exp_shape = (w.batch, w.seqlen, w.nheads, w.headdim) + (() if "o" in which else (w.rank,))
    assert tuple(y.shape) == exp_shape
    check("y", y, y_ref, w.io)
    check_state(fin, f_ref, w.io)
    if "x" in which and w.io == "bf16":
        # the carried x is the rounded x_r of the last token, exactly
        assert np.array_equal(to_np(fin["prev_x"]), ox[:, -1].astype(np.float64))
    return y, fin


# ---------------------------------------------------------------- scans with projections
@pytest.mark.parametrize("which", [("x",), ("z",), ("o",), ("x", "z", "o")])
def test_interleaved_rank_path(which):
    """bf16, rank 4, N = P = 64: the 16-byte interleaved-rank load path."""
    w = custom(batch=2, seqlen=150, nheads=3, headdim=64, dstate=64, rank=4, chunk=16, io="bf16", seed=11)
    run_proj(w, set(which))


@pytest.mark.parametrize("T,P,N,R,Q,io", [
    (97, 32, 32, 2, 32, "bf16"),    # interleaved-rank path, 32 x 32 tiles, R 2
    (70, 64, 128, 8, 16, "bf16"),   # interleaved-rank path, N 128, R 8 (a token's ranks span two lane groups)
    (80, 40, 24, 3, 16, "bf16"),    # element path, R 3 (tokens straddle the waves' rows)
    (80, 40, 24, 3, 16, "f32"),     # element path, fp32
    (64, 16, 16, 2, 32, "f32"),     # element path, fp32 rank 2
    (130, 64, 64, 1, 64, "bf16"),   # rank 1: the projections take the element path
    (45, 5, 6, 5, 16, "f32"),       # odd sizes, ragged tail
])
def test_all_projections_every_path(T, P, N, R, Q, io):
    w = custom(batch=2, seqlen=T, nheads=2, headdim=P, dstate=N, rank=R, chunk=Q, io=io, seed=T + R)
    run_proj(w, {"x", "z", "o"})


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_projections_long_segments(io):
    """Many blocks per sequence: the state kernels expand x too (sub-segments, prefix pass)."""
    w = custom(batch=1, seqlen=2048, nheads=2, headdim=64, dstate=64, rank=2, chunk=32, io=io, seed=5)
    run_proj(w, {"x", "z", "o"})


def test_projections_without_gate_or_state():
    w = custom(batch=2, seqlen=100, nheads=2, headdim=64, dstate=64, rank=4, chunk=16, io="bf16", seed=21)
    run_proj(w, {"x", "o"}, gate_z=False, init=False)


def test_projections_noalloc_matches_workspace_call():
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=200, nheads=2, headdim=64, dstate=64, rank=4, chunk=16, io="bf16", seed=23)
    log(f"case projections noalloc vs workspace call {w}")
    _, _, _, g, params, st0 = proj_case(w, {"x", "z", "o"})
    d = gpu_kwargs(g, params, w)
    args = [d.pop(k) for k in ("x", "B", "C", "dt", "lam", "theta", "A", "D")]
    d["init"] = state_to_dev(st0)
    y1, f1 = m3.m3_scan_mimo(*args, chunk=w.chunk, final=True, **d)
    y2 = torch.empty_like(y1)
    f2 = m3.new_state(w.batch, w.nheads, w.headdim, w.dstate, w.rank)
    m3.m3_scan_noalloc(*args, y=y2, chunk=w.chunk, final=f2, **d)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for k in f1:
        assert torch.equal(f1[k], f2[k]), k


# ---------------------------------------------------------------- decode step with projections
@pytest.mark.parametrize("R,P,N,io", [(4, 64, 64, "bf16"), (1, 64, 64, "f32"), (3, 12, 16, "f32"),
                                      (2, 32, 32, "bf16")])
def test_step_with_projections(R, P, N, io):
    """scan (40 tokens) -> 3 steps -> scan (20 tokens), state in place == one-shot oracle."""
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=63, nheads=2, headdim=P, dstate=N, rank=R, chunk=16, io=io, seed=R * 7 + P)
    log(f"case step with projections {w}")
    inp, ox, o_kw, g, params, st0 = proj_case(w, {"x", "z", "o"})
    y_ref, f_ref = oracle.scan(ox, inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"], inp["D"],
                               init=st0, **o_kw)
    d = gpu_kwargs(g, params, w)
    per_tok = ("x", "B", "C", "dt", "lam", "theta", "z")
    state = state_to_dev(st0)
    pieces, t0 = [], 0
    for kind, n in (("scan", 40), ("step", 3), ("scan", 20)):
        sl = {k: (v[:, t0:t0 + n].contiguous() if k in per_tok else v) for k, v in d.items()}
        if kind == "scan":
            args = [sl.pop(k) for k in ("x", "B", "C", "dt", "lam", "theta", "A", "D")]
            y, _ = m3.m3_scan_mimo(*args, chunk=16, init=state, final=state, **sl)
            pieces.append(y)
        else:
            for k in range(n):
                one = {kk: (vv[:, k:k + 1].contiguous() if kk in per_tok else vv) for kk, vv in sl.items()}
                args = [one.pop(kk) for kk in ("x", "B", "C", "dt", "lam", "theta", "A", "D")]
                pieces.append(m3.m3_step(*args, state, **one))
        t0 += n
    torch.cuda.synchronize()
    y = torch.cat(pieces, dim=1)
    check("y (scan/step/scan)", y, y_ref, io)
    check_state(state, f_ref, io)


# ---------------------------------------------------------------- row-strided inputs
def _strided_views(w, inp, ex, pad_big, pad_f32, with_z=True, contiguous_a=True):
    """Copy the inputs into two in_proj-like buffers (io dtype: z, x, B, C; fp32: dt, lam,
    theta, and a per-token A unless ``contiguous_a``) and return views of them."""
    import torch
    Bsz, T = w.batch, w.seqlen
    big_parts = ([("z", ex["z"])] if with_z else []) + [("x", inp["x"]), ("B", inp["B"]), ("C", inp["C"])]
    f_parts = [("dt", inp["dt"]), ("lam", inp["lam"]), ("theta", inp["theta"])]
    if not contiguous_a:
        f_parts.append(("A", ex["A_tok"]))
    widths = {k: int(np.prod(v.shape[2:])) for k, v in big_parts + f_parts}
    # each part starts on a 16-byte boundary of the row (the library needs aligned base pointers)
    eb = 8 if w.io == "bf16" else 4
    room = {k: -(-widths[k] // eb) * eb for k, _ in big_parts}
    room.update({k: -(-widths[k] // 4) * 4 for k, _ in f_parts})
    Wb = sum(room[k] for k, _ in big_parts) + pad_big
    Wf = sum(room[k] for k, _ in f_parts) + pad_f32
    bt = torch.bfloat16 if w.io == "bf16" else torch.float32
    buf = torch.full((Bsz, T, Wb), float("nan"), dtype=bt, device="cuda")
    fbuf = torch.full((Bsz, T, Wf), float("nan"), dtype=torch.float32, device="cuda")
    views, o = {}, 0
    for k, v in big_parts:
        sl = buf[:, :, o:o + widths[k]]
        sl.copy_(_dev(v.reshape(Bsz, T, -1), w.io, big=True))
        views[k] = sl.unflatten(-1, v.shape[2:])
        o += room[k]
    o = 0
    for k, v in f_parts:
        sl = fbuf[:, :, o:o + widths[k]]
        sl.copy_(_dev(v.reshape(Bsz, T, -1), w.io))
        views[k] = sl.unflatten(-1, v.shape[2:]) if v.ndim > 3 else sl
        o += room[k]
    return views


@pytest.mark.parametrize("T,P,N,R,io,pad_big,pad_f32", [
    (150, 64, 64, 1, "bf16", 8, 4),     # rank-1 16-byte path, 16-byte row strides
    (150, 64, 64, 1, "f32", 4, 4),      # rank-1 16-byte path, fp32
    (90, 64, 64, 4, "bf16", 8, 4),      # interleaved-rank path
    (90, 40, 24, 3, "f32", 4, 0),       # element path
])
def test_strided_inputs_bit_exact(T, P, N, R, io, pad_big, pad_f32):
    """Slices of in_proj-like buffers give bit for bit the contiguous call's results (the same
    kernels run) and match the oracle."""
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=T, nheads=2, headdim=P, dstate=N, rank=R, chunk=16, io=io, seed=T + P)
    log(f"case strided inputs pads ({pad_big}, {pad_f32}) {w}")
    inp, ex = make_inputs(w), make_block_inputs(w)
    st0 = make_state(w, scale=0.4)
    v = _strided_views(w, inp, ex, pad_big, pad_f32, contiguous_a=False)
    assert not v["x"].is_contiguous() and not v["dt"].is_contiguous()
    fn = m3.m3_scan_mimo if R > 1 else m3.m3_scan_siso
    D = _dev(inp["D"], io)
    order = ("x", "B", "C", "dt", "lam", "theta", "A")
    y1, f1 = fn(*(v[k] for k in order), D, chunk=16, z=v["z"], init=state_to_dev(st0), final=True)
    c = {k: t.contiguous() for k, t in v.items()}
    y2, f2 = fn(*(c[k] for k in order), D, chunk=16, z=c["z"], init=state_to_dev(st0), final=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for k in f1:
        assert torch.equal(f1[k], f2[k]), k
    y_ref, f_ref = oracle.scan(inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], ex["A_tok"],
                               inp["D"], init=st0, z=ex["z"])
    check("y", y1, y_ref, io)
    check_state(f1, f_ref, io)


@pytest.mark.parametrize("R,io", [(1, "bf16"), (4, "bf16"), (1, "f32")])
def test_strided_rows_not_16_byte_multiples(R, io):
    """Row strides that are not a multiple of 16 bytes (or B and C rows of different strides)
    take the element path; results match the oracle."""
    import torch
    m3 = _m3()
    w = custom(batch=2, seqlen=120, nheads=2, headdim=64, dstate=64, rank=R, chunk=16, io=io, seed=R + 50)
    log(f"case odd row strides {w}")
    inp, ex = make_inputs(w), make_block_inputs(w)
    v = _strided_views(w, inp, ex, 3, 1)
    # B alone from a buffer of another row length: B and C strides differ
    Bw = int(np.prod(inp["B"].shape[2:]))
    bb = torch.zeros((w.batch, w.seqlen, Bw + 8), dtype=v["B"].dtype, device="cuda")
    bb[:, :, :Bw].copy_(v["B"].reshape(w.batch, w.seqlen, Bw))
    v["B"] = bb[:, :, :Bw].unflatten(-1, inp["B"].shape[2:])
    fn = m3.m3_scan_mimo if R > 1 else m3.m3_scan_siso
    y = fn(v["x"], v["B"], v["C"], v["dt"], v["lam"], v["theta"], _dev(inp["A"], io), _dev(inp["D"], io),
           chunk=16, z=v["z"])
    torch.cuda.synchronize()
    y_ref, _ = oracle.scan(inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"], inp["D"],
                           z=ex["z"])
    check("y", y, y_ref, io)


@pytest.mark.parametrize("R,P,N,io", [(1, 64, 64, "bf16"), (2, 32, 32, "f32")])
def test_step_strided_bit_exact(R, P, N, io):
    """The decode step on slices of in_proj-like rows equals the step on contiguous copies."""
    import torch
    m3 = _m3()
    w = custom(batch=3, seqlen=1, nheads=2, headdim=P, dstate=N, rank=R, chunk=16, io=io, seed=R + 60)
    log(f"case strided step {w}")
    inp, ex = make_inputs(w), make_block_inputs(w)
    st0 = make_state(w, scale=0.4)
    v = _strided_views(w, inp, ex, 8, 4, contiguous_a=False)
    c = {k: t.contiguous() for k, t in v.items()}
    s1, s2 = state_to_dev(st0), state_to_dev(st0)
    order = ("x", "B", "C", "dt", "lam", "theta", "A")
    D = _dev(inp["D"], io)
    y1 = m3.m3_step(*(v[k] for k in order), D, s1, z=v["z"])
    y2 = m3.m3_step(*(c[k] for k in order), D, s2, z=c["z"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for k in s1:
        assert torch.equal(s1[k], s2[k]), k
