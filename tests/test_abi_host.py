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
