"""The allocation-free scan entry point (m3_scan_noalloc, the library's static scratch as
workspace) against the entry point it varies (m3_scan_mimo, any rank; m3_scan_siso at rank
1), through the C ABI: two calls in a row on the same GPU, the second with a smaller input,
each compared element by element, and both compared with the fp64 oracle."""
import numpy as np
import pytest

import oracle
from synth import WORKLOADS, custom, make_inputs, make_norm_params, make_state
from tests.gpu_util import err_metrics, gate, log, oracle_args, state_to_dev, to_dev, to_np

pytestmark = pytest.mark.gpu


def _m3():
    import mamba_selective_scan_amd as m3
    m3.load()
    return m3


def _pair(m3, w, inp, npar, st0, *, half_split=False):
    """(noalloc outputs, reference entry point outputs) for one input."""
    import torch
    d = to_dev(inp, w.io)
    pd = {k: torch.from_numpy(v).cuda() for k, v in npar.items()}
    args = (d["x"], d["B"], d["C"], d["dt"], d["lam"], d["theta"], d["A"], d["D"])
    R, NR = w.rank, w.dstate // 2
    y_na = torch.empty_like(d["x"])
    fin_na = m3.new_state(w.batch, w.nheads, w.headdim, w.dstate, R, "cuda", NR)
    m3.m3_scan_noalloc(*args, y=y_na, chunk=w.chunk, init=state_to_dev(st0), final=fin_na,
                       half_split=half_split, **pd)
    ref = m3.m3_scan_mimo if R > 1 else m3.m3_scan_siso
    y_ref, fin_ref = ref(*args, chunk=w.chunk, init=state_to_dev(st0), final=True, half_split=half_split, **pd)
    torch.cuda.synchronize()
    return (y_na, fin_na), (y_ref, fin_ref)


def _compare(name, got, ref, w, y_oracle):
    (y_na, fin_na), (y_ref, fin_ref) = got, ref
    raw, _ = err_metrics(to_np(y_na), to_np(y_ref), "f32")
    log(f"  {name}: noalloc vs workspace entry point max|diff|/rms = {raw:.3e}")
    assert np.array_equal(to_np(y_na), to_np(y_ref)), name
    for k in fin_ref:
        assert np.array_equal(to_np(fin_na[k]), to_np(fin_ref[k])), f"{name} final {k}"
    _, comp = err_metrics(to_np(y_na), y_oracle, w.io)
    log(f"  {name}: noalloc vs oracle compute err = {comp:.3e} (gate {gate(w.io):.0e})")
    assert comp <= gate(w.io)


@pytest.mark.parametrize("rank", [1, 4])
def test_noalloc_two_calls_second_smaller(rank):
    m3 = _m3()
    big = WORKLOADS[1] if rank == 1 else WORKLOADS[2]
    small = custom(batch=2, seqlen=333, nheads=3, headdim=64, dstate=64, rank=rank, chunk=big.chunk,
                   io="bf16", seed=77)
    for w, tag in ((big, "first (full workload)"), (small, "second (smaller)")):
        log(f"case noalloc rank {rank} {tag}: {w}")
        inp = make_inputs(w)
        npar = make_norm_params(w)
        st0 = make_state(w, scale=0.3)
        y_or, _ = oracle.scan(*oracle_args(inp), init=st0, **npar)
        got, ref = _pair(m3, w, inp, npar, st0)
        _compare(tag, got, ref, w, y_or)


def test_noalloc_half_split_and_fp32():
    m3 = _m3()
    for w, hs in ((custom(batch=2, seqlen=500, nheads=2, headdim=64, dstate=64, io="bf16", seed=5), True),
                  (custom(batch=1, seqlen=130, nheads=2, headdim=24, dstate=6, rank=3, chunk=16, io="f32",
                          seed=6), False)):
        log(f"case noalloc half_split={hs} {w}")
        inp = make_inputs(w)
        npar = make_norm_params(w)
        st0 = make_state(w, scale=0.3)
        y_or, _ = oracle.scan(*oracle_args(inp), init=st0, half_split=hs, **npar)
        got, ref = _pair(m3, w, inp, npar, st0, half_split=hs)
        _compare("call", got, ref, w, y_or)


def test_noalloc_rejects_oversized_shape():
    """A shape whose workspace exceeds the static scratch (the half-split pairing's permuted
    copies of B and C, 2 x 67 MB) is rejected before any launch."""
    import torch
    m3 = _m3()
    log("case noalloc oversized shape")
    Bz, T, H, P, N = 16, 4096, 16, 64, 64
    x = torch.zeros((Bz, T, H, P), dtype=torch.bfloat16, device="cuda")
    Bm = torch.zeros((Bz, T, H, N), dtype=torch.bfloat16, device="cuda")
    f = lambda *sh: torch.zeros(sh, dtype=torch.float32, device="cuda")
    y = torch.full_like(x, 3.0)
    with pytest.raises(RuntimeError, match="static scratch"):
        m3.m3_scan_noalloc(x, Bm, Bm, f(Bz, T, H), f(Bz, T, H), f(Bz, T, H, N // 2), f(H), f(H), y=y,
                           half_split=True)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())  # nothing ran
