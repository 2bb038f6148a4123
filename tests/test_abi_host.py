"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, sizes the workspace, and rejects bad arguments before any HIP call.
No kernel is launched here (runs without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmamba3.h")


def _lib():
    import mamba_selective_scan_amd as m3
    if not os.path.exists(m3.lib_path):
        from mamba_selective_scan_amd import build
        build.build(verbose=False)
    return m3, m3.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(m3_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    m3, lib = _lib()
    names = declared_functions()
    assert set(names) >= {"m3_scan_siso", "m3_scan_mimo", "m3_step", "m3_scan_workspace_bytes",
                          "m3_status_str", "m3_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.m3_version().decode().count(".") == 2


def _shape(m3, **kw):
    base = dict(batch=4, seqlen=2048, nheads=16, headdim=64, dstate=64, rank=1, chunk=64,
                io=m3.M3_BF16, flags=m3.M3_FLAG_BCNORM, norm_eps=1e-5)
    base.update(kw)
    return m3.Shape(**base)


def test_workspace_bytes():
    m3, lib = _lib()
    s = _shape(m3)
    ws = m3.m3_scan_workspace_bytes(s)
    state = 16 * 64 * 64 * 4  # one (N x P) fp32 state per head
    # per (batch, head): one state per state sub-segment (at most 64) and one incoming state
    # per output segment (at most 16)
    assert 4 * state <= ws <= 4 * (64 + 16) * state * 1.1
    assert m3.m3_scan_workspace_bytes(_shape(m3, seqlen=0)) == 0
    assert m3.m3_scan_workspace_bytes(_shape(m3, dstate=63)) == 0
    # a single block needs a single segment per sequence (and no sub-segments)
    one = m3.m3_scan_workspace_bytes(_shape(m3, seqlen=10))
    assert 4 * state <= one < 4 * 2 * state * 1.1


def _fake_inputs(m3):
    # host addresses that are 16-byte aligned; never dereferenced (calls fail validation first)
    buf = ctypes.create_string_buffer(4096)
    base = (ctypes.addressof(buf) + 15) // 16 * 16
    ptrs = {n: ctypes.c_void_p(base) for n in ("x", "Bm", "Cm", "dt", "lam", "theta", "A", "D")}
    return buf, ptrs


def _call_scan(m3, lib, s, inp_over=None, y=True, ws_bytes=None, init=None, fin=None, mimo=False):
    buf, ptrs = _fake_inputs(m3)
    if inp_over:
        ptrs.update(inp_over)
    inp = m3._Inputs(**ptrs)
    ws = ctypes.c_void_p(ptrs["x"].value)
    nbytes = ws_bytes if ws_bytes is not None else m3.m3_scan_workspace_bytes(s) + 1024
    f = lib.m3_scan_mimo if mimo else lib.m3_scan_siso
    rc = f(ctypes.byref(s), ctypes.byref(inp), ptrs["x"] if y else None,
           ctypes.byref(init) if init is not None else None,
           ctypes.byref(fin) if fin is not None else None, ws, ctypes.c_size_t(nbytes), None)
    return rc


@pytest.mark.parametrize("kw,code", [
    (dict(dstate=63), 1),          # odd N
    (dict(dstate=0), 1),
    (dict(rank=0), 1),
    (dict(nheads=0), 1),
    (dict(headdim=0), 1),
    (dict(batch=-1), 1),
    (dict(seqlen=-5), 1),
    (dict(io=7), 1),
    (dict(flags=0x40), 1),         # unknown flag
    (dict(flags=0x21, rank=2), 1),  # half-split SISO call with rank 2
    (dict(flags=0x80000001), 1),
    (dict(flags=3, rope_pairs=33), 1),   # more rotated pairs than N/2
    (dict(flags=3, rope_pairs=-1), 1),
    (dict(rank=2), 1),             # SISO call with rank 2
    (dict(dstate=130), 2),         # N > 128
    (dict(headdim=129), 2),
    (dict(chunk=48), 2),
    (dict(chunk=8), 2),
])
def test_invalid_shapes(kw, code):
    m3, lib = _lib()
    s = _shape(m3, **kw)
    assert _call_scan(m3, lib, s) == code


def test_invalid_pointers_and_workspace():
    m3, lib = _lib()
    s = _shape(m3)
    assert _call_scan(m3, lib, s, inp_over={"dt": None}) == 1
    assert _call_scan(m3, lib, s, inp_over={"theta": None}) == 1
    _, ptrs = _fake_inputs(m3)
    mis = ctypes.c_void_p(ptrs["x"].value + 2)
    assert _call_scan(m3, lib, s, inp_over={"Bm": mis}) == 1     # misaligned
    assert _call_scan(m3, lib, s, y=False) == 1                  # no output
    assert _call_scan(m3, lib, s, ws_bytes=100) == 3             # short workspace
    half = m3._State(h=ptrs["x"], prev_B=None, prev_x=ptrs["x"], angle=ptrs["x"])
    assert _call_scan(m3, lib, s, init=half) == 1                # incomplete state


def test_option_pointers():
    m3, lib = _lib()
    _, ptrs = _fake_inputs(m3)
    mis = ctypes.c_void_p(ptrs["x"].value + 4)
    s = _shape(m3, flags=m3.M3_FLAG_BCNORM | m3.M3_FLAG_DT_SOFTPLUS)
    assert _call_scan(m3, lib, s, inp_over={"dt_bias": mis}) == 1   # misaligned dt bias
    assert _call_scan(m3, lib, s, inp_over={"z": mis}) == 1         # misaligned gate input
    # no rotated pair: theta and the state's angle may be NULL (the call then stops at the
    # short workspace, after every pointer check)
    s0 = _shape(m3, flags=m3.M3_FLAG_BCNORM | m3.M3_FLAG_PARTIAL_ROPE, rope_pairs=0)
    st = m3._State(h=ptrs["x"], prev_B=ptrs["x"], prev_x=ptrs["x"], angle=None)
    assert _call_scan(m3, lib, s0, inp_over={"theta": None}, init=st, ws_bytes=100) == 3
    s1 = _shape(m3, flags=m3.M3_FLAG_BCNORM | m3.M3_FLAG_PARTIAL_ROPE, rope_pairs=1)
    assert _call_scan(m3, lib, s1, inp_over={"theta": None}, ws_bytes=100) == 1
    assert _call_scan(m3, lib, s1, init=st, ws_bytes=100) == 1


def test_half_split_workspace():
    """The half-split pairing needs room for the N-permuted copies of B, C (and, for the
    gradient call, of their gradients) beside the plain call's workspace; a workspace of the
    plain size is short (checked before any launch)."""
    m3, lib = _lib()
    s = _shape(m3)
    sh = _shape(m3, flags=m3.M3_FLAG_BCNORM | m3.M3_FLAG_HALF_SPLIT)
    plain, split = lib.m3_scan_workspace_bytes(ctypes.byref(s)), lib.m3_scan_workspace_bytes(ctypes.byref(sh))
    bc = 2 * s.batch * s.seqlen * s.nheads * s.dstate * s.rank * 2  # bf16 copies of B and C
    assert split >= plain + bc
    assert _call_scan(m3, lib, sh, ws_bytes=plain) == 3
    bplain = lib.m3_scan_bwd_workspace_bytes(ctypes.byref(s))
    bsplit = lib.m3_scan_bwd_workspace_bytes(ctypes.byref(sh))
    assert bsplit >= bplain + 2 * bc


def test_mimo_limits():
    m3, lib = _lib()
    assert _call_scan(m3, lib, _shape(m3, rank=9, chunk=16), mimo=True) == 2   # R > 8
    assert _call_scan(m3, lib, _shape(m3, rank=4, chunk=64), mimo=True) == 2   # 256 rows
    assert _call_scan(m3, lib, _shape(m3, rank=0, chunk=16), mimo=True) == 1


def test_step_validation():
    m3, lib = _lib()
    _, ptrs = _fake_inputs(m3)
    inp = m3._Inputs(**ptrs)
    st = m3._State(h=ptrs["x"], prev_B=ptrs["x"], prev_x=ptrs["x"], angle=ptrs["x"])
    s = _shape(m3, seqlen=2)
    assert lib.m3_step(ctypes.byref(s), ctypes.byref(inp), ptrs["x"], ctypes.byref(st), None) == 1
    s = _shape(m3, seqlen=1)
    assert lib.m3_step(ctypes.byref(s), ctypes.byref(inp), ptrs["x"], None, None) == 1
    s = _shape(m3, seqlen=1, dstate=5)
    assert lib.m3_step(ctypes.byref(s), ctypes.byref(inp), ptrs["x"], ctypes.byref(st), None) == 1


def test_status_strings():
    m3, lib = _lib()
    for code, tag in ((0, "M3_OK"), (1, "M3_EINVAL"), (2, "M3_EUNSUPPORTED"), (3, "M3_EWORKSPACE"),
                      (4, "M3_EHIP")):
        assert m3.m3_status_str(code).startswith(tag)
    assert "unknown" in m3.m3_status_str(99)


def test_half_split_checks_before_any_launch():
    """A half-split call permutes B, C and the state into the workspace before the scan
    kernels run; every argument check (output pointer, workspace alignment, the gate's
    gradient) comes before the first of those launches, so on this GPU-less host a bad
    argument reports M3_EINVAL, not a launch failure."""
    m3, lib = _lib()
    sh = _shape(m3, flags=m3.M3_FLAG_BCNORM | m3.M3_FLAG_HALF_SPLIT, seqlen=64)
    assert _call_scan(m3, lib, sh, y=False) == 1                      # no output
    _, ptrs = _fake_inputs(m3)
    inp = m3._Inputs(**ptrs)
    mis = ctypes.c_void_p(ptrs["x"].value + 8)
    big = m3.m3_scan_workspace_bytes(sh) + 4096
    rc = lib.m3_scan_siso(ctypes.byref(sh), ctypes.byref(inp), ptrs["x"], None, None, mis,
                          ctypes.c_size_t(big), None)
    assert rc == 1                                                    # misaligned workspace
    # a gated gradient call without dz
    ptrs_z = dict(ptrs, z=ptrs["x"])
    inz = m3._Inputs(**ptrs_z)
    gr = m3._Grads(dx=ptrs["x"])
    bws = lib.m3_scan_bwd_workspace_bytes(ctypes.byref(sh)) + 4096
    rc = lib.m3_scan_bwd(ctypes.byref(sh), ctypes.byref(inz), ptrs["x"], None, None, ctypes.byref(gr), None,
                         ptrs["x"], ctypes.c_size_t(bws), None)
    assert rc == 1


def test_half_split_empty_needs_no_workspace():
    """With no tokens (or no batch) a call only copies the state, whatever the pairing: the
    workspace size is 0 for the scans and the gradient call."""
    m3, lib = _lib()
    for kw in (dict(seqlen=0), dict(batch=0)):
        sh = _shape(m3, flags=m3.M3_FLAG_BCNORM | m3.M3_FLAG_HALF_SPLIT, **kw)
        assert lib.m3_scan_workspace_bytes(ctypes.byref(sh)) == 0
        assert lib.m3_scan_bwd_workspace_bytes(ctypes.byref(sh)) == 0
        s = _shape(m3, **kw)
        assert lib.m3_scan_workspace_bytes(ctypes.byref(s)) == 0
    # B == 0 with no workspace at all succeeds without touching the device
    sh = _shape(m3, flags=m3.M3_FLAG_BCNORM | m3.M3_FLAG_HALF_SPLIT, batch=0)
    _, ptrs = _fake_inputs(m3)
    inp = m3._Inputs(**ptrs)
    assert lib.m3_scan_siso(ctypes.byref(sh), ctypes.byref(inp), ptrs["x"], None, None, None,
                            ctypes.c_size_t(0), None) == 0


def test_noalloc_rejects_shapes_beyond_static_scratch():
    """m3_scan_noalloc checks every argument, then that the shape's workspace fits the
    library's static scratch, before touching the device (this host has none)."""
    m3, lib = _lib()
    _, ptrs = _fake_inputs(m3)
    inp = m3._Inputs(**ptrs)
    # the half-split pairing puts permuted copies of B and C into the workspace: 2 x 67 MB here
    big = _shape(m3, batch=16, seqlen=4096, flags=m3.M3_FLAG_BCNORM | m3.M3_FLAG_HALF_SPLIT)
    assert m3.m3_scan_workspace_bytes(big) > m3.M3_STATIC_SCRATCH_BYTES
    assert lib.m3_scan_noalloc(ctypes.byref(big), ctypes.byref(inp), ptrs["x"], None, None, None) == 3
    assert lib.m3_scan_noalloc(ctypes.byref(_shape(m3, dstate=63)), ctypes.byref(inp), ptrs["x"], None, None,
                               None) == 1
    assert lib.m3_scan_noalloc(ctypes.byref(_shape(m3)), ctypes.byref(inp), None, None, None, None) == 1
    text = open(HEADER).read()
    assert f"#define M3_STATIC_SCRATCH_BYTES (64u << 20)" in text and m3.M3_STATIC_SCRATCH_BYTES == 64 << 20


def test_projection_and_stride_checks():
    """MIMO projections and row strides are checked before any launch: a projection on the
    SISO entry point, mimo_z without a gate input or a misaligned vector is M3_EINVAL; a row
    stride shorter than its row M3_EINVAL, one of 2^24 or more M3_EUNSUPPORTED; strided B or C
    with the half-split pairing, and strides or projections on the gradient call, are
    M3_EUNSUPPORTED.  Valid strides pass every check (the call then stops at the short
    workspace, M3_EWORKSPACE)."""
    m3, lib = _lib()
    _, ptrs = _fake_inputs(m3)
    mis = ctypes.c_void_p(ptrs["x"].value + 4)
    s1 = _shape(m3)
    s4 = _shape(m3, rank=4, chunk=16)
    assert _call_scan(m3, lib, s1, inp_over={"mimo_x": ptrs["x"]}) == 1
    assert _call_scan(m3, lib, s4, inp_over={"mimo_z": ptrs["x"]}, mimo=True) == 1
    assert _call_scan(m3, lib, s4, inp_over={"mimo_z": ptrs["x"], "z": ptrs["x"]}, mimo=True, ws_bytes=100) == 3
    assert _call_scan(m3, lib, s4, inp_over={"mimo_o": mis}, mimo=True) == 1
    assert _call_scan(m3, lib, s4, inp_over={"mimo_x": ptrs["x"], "mimo_o": ptrs["x"]}, mimo=True,
                      ws_bytes=100) == 3
    H, P, N = s1.nheads, s1.headdim, s1.dstate
    assert _call_scan(m3, lib, s1, inp_over={"x_stride": H * P - 1}) == 1
    assert _call_scan(m3, lib, s1, inp_over={"theta_stride": H * N // 2 - 4}) == 1
    assert _call_scan(m3, lib, s1, inp_over={"dt_stride": 1 << 24}) == 2
    assert _call_scan(m3, lib, s1, inp_over={"z_stride": -1}) == 1
    ok = {"x_stride": 2 * H * P + 8, "B_stride": 2 * H * P + 8, "C_stride": 2 * H * P + 8, "dt_stride": H + 3,
          "lam_stride": H + 3, "theta_stride": H * N // 2 + 1, "z_stride": 2 * H * P + 8}
    assert _call_scan(m3, lib, s1, inp_over=ok, ws_bytes=100) == 3
    # a MIMO call's rank-free x (mimo_x) has rows of H * P: a stride of H * P is valid there
    assert _call_scan(m3, lib, s4, inp_over={"mimo_x": ptrs["x"], "x_stride": H * P}, mimo=True, ws_bytes=100) == 3
    assert _call_scan(m3, lib, s4, inp_over={"x_stride": H * P}, mimo=True) == 1
    sh = _shape(m3, flags=m3.M3_FLAG_BCNORM | m3.M3_FLAG_HALF_SPLIT)
    assert _call_scan(m3, lib, sh, inp_over={"C_stride": H * N + 8}) == 2
    assert _call_scan(m3, lib, sh, inp_over={"x_stride": H * P + 8}, ws_bytes=100) == 3
    gr = m3._Grads(dx=ptrs["x"])
    bws = lib.m3_scan_bwd_workspace_bytes(ctypes.byref(s1)) + 4096
    for over in ({"x_stride": H * P + 8}, {"dt_stride": H + 1}):
        inp = m3._Inputs(**dict(ptrs, **over))
        rc = lib.m3_scan_bwd(ctypes.byref(s1), ctypes.byref(inp), ptrs["x"], None, None, ctypes.byref(gr), None,
                             ptrs["x"], ctypes.c_size_t(bws), None)
        assert rc == 2, over
    inp = m3._Inputs(**dict(ptrs, mimo_x=ptrs["x"]))
    rc = lib.m3_scan_bwd(ctypes.byref(s4), ctypes.byref(inp), ptrs["x"], None, None, ctypes.byref(gr), None,
                         ptrs["x"], ctypes.c_size_t(lib.m3_scan_bwd_workspace_bytes(ctypes.byref(s4)) + 4096), None)
    assert rc == 2
    # the decode step: a short stride, and mimo_z without z
    st = m3._State(h=ptrs["x"], prev_B=ptrs["x"], prev_x=ptrs["x"], angle=ptrs["x"])
    s1t = _shape(m3, seqlen=1)
    inp = m3._Inputs(**dict(ptrs, B_stride=N - 2))
    assert lib.m3_step(ctypes.byref(s1t), ctypes.byref(inp), ptrs["x"], ctypes.byref(st), None) == 1
    inp = m3._Inputs(**dict(ptrs, mimo_z=ptrs["x"]))
    s4t = _shape(m3, seqlen=1, rank=4)
    assert lib.m3_step(ctypes.byref(s4t), ctypes.byref(inp), ptrs["x"], ctypes.byref(st), None) == 1


def test_binding_row_strides():
    """The binding passes a slice of a wider buffer (contiguous token rows, evenly spaced) as
    a pointer and a row stride, and refuses other non-contiguous layouts (host tensors only;
    nothing is launched)."""
    import torch
    m3, _ = _lib()
    Bsz, T, H, P = 2, 5, 3, 4
    buf = torch.zeros(Bsz, T, 2 * H * P + 6)
    x = buf[:, :, H * P:2 * H * P].unflatten(-1, (H, P))
    assert m3._need(x, "x", torch.float32, x.device, (Bsz, T, H, P), rows=True) == 2 * H * P + 6
    assert m3._need(x.contiguous(), "x", torch.float32, x.device, (Bsz, T, H, P), rows=True) == 0
    one = buf[:, :1, :H * P].unflatten(-1, (H, P))  # one token: rows b are a batch stride apart
    assert m3._need(one, "x", torch.float32, x.device, (Bsz, 1, H, P), rows=True) == T * (2 * H * P + 6)
    with pytest.raises(ValueError):
        m3._need(x.transpose(2, 3), "x", torch.float32, x.device, None, rows=True)   # rows not contiguous
    with pytest.raises(ValueError):
        m3._need(buf[:, ::2, :H * P].unflatten(-1, (H, P))[:, :, :, :2], "x", torch.float32, x.device, None,
                 rows=True)
    with pytest.raises(ValueError):
        m3._need(x, "x", torch.float32, x.device, (Bsz, T, H, P))   # rows=False: contiguous only
    # batch rows not T row strides apart
    wide = torch.zeros(Bsz, T + 1, H * P)[:, :T].unflatten(-1, (H, P))
    assert m3._row_stride(wide) is None


def test_binding_gradient_call_takes_contiguous_inputs():
    """The gradient call's input block refuses row-strided slices (host tensors; nothing runs)."""
    import torch
    m3, _ = _lib()
    Bsz, T, H, P, N = 1, 4, 2, 8, 8
    s = m3.Shape(Bsz, T, H, P, N, 1, 16, m3.M3_F32, m3.M3_FLAG_BCNORM, 1e-5)
    f = lambda *sh: torch.zeros(sh)
    args = dict(x=f(Bsz, T, H, P), B=f(Bsz, T, H, N), C=f(Bsz, T, H, N), dt=f(Bsz, T, H), lam=f(Bsz, T, H),
                theta=f(Bsz, T, H, N // 2), A=f(H), D=f(H))
    pos = lambda a: [a[k] for k in ("x", "B", "C", "dt", "lam", "theta", "A", "D")]
    inp = m3._inputs(s, *pos(args), None, None, None, None, False, strided=False)
    assert inp.x_stride == 0 and inp.dt_stride == 0
    args["dt"] = f(Bsz, T, H + 2)[:, :, :H]
    assert m3._inputs(s, *pos(args), None, None, None, None, False).dt_stride == H + 2
    with pytest.raises(ValueError):
        m3._inputs(s, *pos(args), None, None, None, None, False, strided=False)


def test_debug_checks_unsupported_in_release_build():
    """m3_debug_checks reads the device-side check counters of a -DM3_DEBUG build; the release
    library checks nothing and says so (M3_EUNSUPPORTED) without touching a device."""
    m3, lib = _lib()
    lib.m3_debug_checks.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert lib.m3_debug_checks(None, None) == 2
