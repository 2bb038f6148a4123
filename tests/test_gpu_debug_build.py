"""The debug build (-DM3_DEBUG, libmamba3_debug.so): its device-side index checks hold on
ragged shapes of every kernel path (rank-1 16-byte, element, interleaved-rank, long segments
with the prefix pass, MIMO projections, strided rows, half-split, decode step, gradients),
and its results still match the fp64 oracle.  A failed check is counted on the device (no
fault) and read back with m3_debug_checks.  Skipped when the debug library is not built
(python -m mamba_selective_scan_amd.build --debug).
"""
import ctypes
import os

import numpy as np
import pytest

import oracle
from synth import custom, make_block_inputs, make_inputs, make_state
from tests.gpu_util import err_metrics, gate, log, state_to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m3dbg():
    import mamba_selective_scan_amd as m3
    from mamba_selective_scan_amd import build as b
    if not os.path.exists(b.DEBUG_LIB):
        pytest.skip("libmamba3_debug.so not built")
    saved = (m3._lib, m3.lib_path)
    m3._lib, m3.lib_path = None, b.DEBUG_LIB
    lib = m3.load()
    lib.m3_debug_checks.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    lib.m3_debug_checks.restype = ctypes.c_int
    yield m3, lib
    m3._lib, m3.lib_path = saved


def _checks(lib):
    failed, line = ctypes.c_uint32(0), ctypes.c_uint32(0)
    assert lib.m3_debug_checks(ctypes.byref(failed), ctypes.byref(line)) == 0
    return failed.value, line.value


def _dev(a, io, big=False):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.to(torch.bfloat16) if (big and io == "bf16") else t).cuda()


@pytest.mark.parametrize("T,P,N,R,Q,io,opts", [
    (300, 64, 64, 1, 64, "bf16", ()),                  # rank-1 16-byte path, ragged tail
    (77, 5, 6, 1, 16, "f32", ("gate",)),               # element path, odd sizes
    (97, 64, 64, 4, 16, "bf16", ("gate",)),            # interleaved-rank path
    (61, 40, 24, 3, 16, "f32", ()),                    # element path, R 3
    (2100, 32, 32, 1, 16, "bf16", ()),                 # many blocks: sub-segments and the prefix pass
    (130, 64, 64, 2, 32, "bf16", ("proj",)),           # MIMO projections
    (150, 64, 64, 1, 64, "bf16", ("half",)),           # half-split pairing
])
def test_debug_checks_scan_and_gradients(m3dbg, T, P, N, R, Q, io, opts):
    import torch
    m3, lib = m3dbg
    _checks(lib)  # clear
    w = custom(batch=2, seqlen=T, nheads=2, headdim=P, dstate=N, rank=R, chunk=Q, io=io, seed=T + N)
    log(f"case debug build {opts} {w}")
    inp, ex = make_inputs(w), make_block_inputs(w)
    st0 = make_state(w, scale=0.3)
    kw, okw = {}, {}
    if "gate" in opts:
        kw["z"], okw["z"] = _dev(ex["z"], io, True), ex["z"]
    if "half" in opts:
        kw["half_split"] = okw["half_split"] = True
    x = inp["x"]
    if "proj" in opts:
        rng = np.random.default_rng(3)
        mo = rng.uniform(-1, 1, (w.nheads, R, P)).astype(np.float32)
        kw["mimo_o"], okw["mimo_o"] = _dev(mo, io), mo
    d = {k: _dev(v, io, k in ("x", "B", "C")) for k, v in inp.items()}
    fn = m3.m3_scan_mimo if R > 1 else m3.m3_scan_siso
    y, fin = fn(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], chunk=Q,
                init=state_to_dev(st0), final=True, **kw)
    torch.cuda.synchronize()
    failed, line = _checks(lib)
    assert failed == 0, f"{failed} failed device checks, last at line {line}"
    y_ref, _ = oracle.scan(x, inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"], inp["D"],
                           init=st0, **okw)
    raw, comp = err_metrics(to_np(y), y_ref, io)
    assert comp <= gate(io), comp
    if "proj" not in opts:
        g = m3.m3_scan_bwd(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"],
                           torch.ones_like(y), init=state_to_dev(st0), **kw)
        torch.cuda.synchronize()
        assert np.isfinite(to_np(g["x"])).all()
        failed, line = _checks(lib)
        assert failed == 0, f"gradients: {failed} failed device checks, last at line {line}"


@pytest.mark.parametrize("R,P,N,io", [(1, 64, 64, "bf16"), (3, 12, 16, "f32")])
def test_debug_checks_step(m3dbg, R, P, N, io):
    import torch
    m3, lib = m3dbg
    _checks(lib)
    w = custom(batch=3, seqlen=1, nheads=2, headdim=P, dstate=N, rank=R, chunk=16, io=io, seed=R + 70)
    log(f"case debug build step {w}")
    inp = make_inputs(w)
    st0 = make_state(w, scale=0.3)
    d = {k: _dev(v, io, k in ("x", "B", "C")) for k, v in inp.items()}
    st = state_to_dev(st0)
    y = m3.m3_step(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"], st)
    torch.cuda.synchronize()
    failed, line = _checks(lib)
    assert failed == 0, f"{failed} failed device checks, last at line {line}"
    y_ref, _ = oracle.scan(inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"], inp["D"],
                           init=st0)
    assert err_metrics(to_np(y), y_ref, io)[1] <= gate(io)
