"""Python binding of libmamba3 (Mamba-3 trapezoidal selective scan on MI355X).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libmamba3.so``; this module checks tensor dtypes/devices/contiguity, builds
the C structs, allocates outputs and workspace with torch, and passes raw
device pointers and the current HIP stream to the C ABI
(``include/libmamba3.h``).  The functions carry the C names:

    m3_scan_siso, m3_scan_mimo, m3_step, m3_scan_workspace_bytes, m3_status_str

There is no fallback: if the library is missing or a call fails, a
RuntimeError is raised.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

__all__ = ["m3_scan_siso", "m3_scan_mimo", "m3_step", "m3_scan_bwd", "m3_scan_noalloc", "m3_scan_workspace_bytes",
           "m3_scan_bwd_workspace_bytes",
           "m3_status_str", "Shape", "M3_F32", "M3_BF16", "M3_FLAG_BCNORM", "M3_FLAG_PARTIAL_ROPE",
           "M3_FLAG_A_PER_TOKEN", "M3_FLAG_DT_SOFTPLUS", "M3_FLAG_LAM_SIGMOID", "M3_FLAG_HALF_SPLIT", "lib_path",
           "load"]

M3_F32, M3_BF16 = 0, 1
M3_FLAG_BCNORM = 1 << 0
M3_FLAG_PARTIAL_ROPE = 1 << 1
M3_FLAG_A_PER_TOKEN = 1 << 2
M3_FLAG_DT_SOFTPLUS = 1 << 3
M3_FLAG_LAM_SIGMOID = 1 << 4
M3_FLAG_HALF_SPLIT = 1 << 5
M3_STATIC_SCRATCH_BYTES = 64 << 20
_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmamba3.so")


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("norm_eps", ctypes.c_float),
                ("rope_pairs", ctypes.c_int32)]


_ROW_STRIDED = ("x", "B", "C", "dt", "lam", "theta", "A", "z")


class _Inputs(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_void_p) for n in
                 ("x", "Bm", "Cm", "dt", "lam", "theta", "A", "D",
                  "b_norm_w", "c_norm_w", "b_bias", "c_bias", "dt_bias", "z",
                  "mimo_x", "mimo_z", "mimo_o")] +
                [(n + "_stride", ctypes.c_int64) for n in _ROW_STRIDED])


class _State(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("h", "prev_B", "prev_x", "angle")]


class _Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dB", "dC", "ddt", "dlam", "dtheta", "dA", "dD", "db_norm_w", "dc_norm_w",
                 "db_bias", "dc_bias", "ddt_bias", "dz")]


_lib = None


def load():
    """Load libmamba3.so (built in-tree by ``mamba_selective_scan_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"libmamba3.so not built ({lib_path}); run "
                               "`python -m mamba_selective_scan_amd.build`")
        lib = ctypes.CDLL(lib_path)
        P = ctypes.POINTER
        lib.m3_scan_workspace_bytes.argtypes = [P(Shape)]
        lib.m3_scan_workspace_bytes.restype = ctypes.c_size_t
        for name in ("m3_scan_siso", "m3_scan_mimo"):
            f = getattr(lib, name)
            f.argtypes = [P(Shape), P(_Inputs), ctypes.c_void_p, P(_State), P(_State),
                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
            f.restype = ctypes.c_int
        lib.m3_scan_noalloc.argtypes = [P(Shape), P(_Inputs), ctypes.c_void_p, P(_State), P(_State),
                                        ctypes.c_void_p]
        lib.m3_scan_noalloc.restype = ctypes.c_int
        lib.m3_step.argtypes = [P(Shape), P(_Inputs), ctypes.c_void_p, P(_State), ctypes.c_void_p]
        lib.m3_step.restype = ctypes.c_int
        lib.m3_scan_bwd_workspace_bytes.argtypes = [P(Shape)]
        lib.m3_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.m3_scan_bwd.argtypes = [P(Shape), P(_Inputs), ctypes.c_void_p, P(_State), P(_State), P(_Grads),
                                    P(_State), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.m3_scan_bwd.restype = ctypes.c_int
        lib.m3_status_str.argtypes = [ctypes.c_int]
        lib.m3_status_str.restype = ctypes.c_char_p
        lib.m3_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def m3_status_str(code: int) -> str:
    return load().m3_status_str(int(code)).decode()


def _check(code: int, what: str):
    if code != 0:
        raise RuntimeError(f"{what}: {m3_status_str(code)}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, device, shape=None, rows=False):
    """Check a tensor argument.  With ``rows`` the tensor [B, T, ...] may be a slice of a wider
    buffer: each token's row is contiguous and rows b*T + t are a fixed stride apart; the row
    stride in elements is returned (0 when contiguous)."""
    if t is None:
        return None if not rows else 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.is_contiguous():
        return 0 if rows else t
    if rows and t.dim() >= 3:
        rs = _row_stride(t)
        if rs is not None:
            return rs
        raise ValueError(f"{name}: each token's row must be contiguous, rows evenly spaced")
    raise ValueError(f"{name} must be contiguous")


def _row_stride(t):
    """Elements between consecutive token rows of [B, T, ...] with contiguous rows, or None."""
    Bsz, T = t.shape[0], t.shape[1]
    inner = 1
    for d in range(t.dim() - 1, 1, -1):
        if t.shape[d] != 1 and t.stride(d) != inner:
            return None
        inner *= t.shape[d]
    rs = t.stride(1) if T > 1 else (t.stride(0) if Bsz > 1 else inner)
    if T > 1 and Bsz > 1 and t.stride(0) != rs * T:
        return None
    return rs if rs >= inner else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_on(stream):
    """Context under which a call's outputs and workspace are allocated: the stream the
    kernels run on.  The caching allocator then reuses a block freed here (the workspace,
    released when the call returns) only for later work ordered on that same stream, never
    while the kernels may still read or write it."""
    if stream is None:
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def _shape_of(x, B, chunk, bcnorm, eps, mimo, opts):
    io = {torch.float32: M3_F32, torch.bfloat16: M3_BF16}.get(x.dtype)
    if io is None:
        raise TypeError("x must be float32 or bfloat16")
    if mimo:
        if B.dim() != 5:
            raise ValueError("MIMO B must be [B, T, H, N, R]")
        R = B.shape[4]
        if opts.get("mimo_x") is not None:
            if x.dim() != 4:
                raise ValueError("x must be [B, T, H, P] with mimo_x")
            Bsz, T, H, P = x.shape
        else:
            if x.dim() != 5:
                raise ValueError("MIMO x must be [B, T, H, P, R]")
            Bsz, T, H, P, R = x.shape
        N = B.shape[3]
    else:
        if x.dim() != 4:
            raise ValueError("SISO x must be [B, T, H, P]")
        Bsz, T, H, P = x.shape
        R = 1
        N = B.shape[3]
    flags = M3_FLAG_BCNORM if bcnorm else 0
    nr = opts.get("rope_pairs")
    if nr is not None:
        flags |= M3_FLAG_PARTIAL_ROPE
    A = opts.get("A")
    if A is not None and A.dim() == 3:
        flags |= M3_FLAG_A_PER_TOKEN
    if opts.get("dt_softplus"):
        flags |= M3_FLAG_DT_SOFTPLUS
    if opts.get("lam_sigmoid"):
        flags |= M3_FLAG_LAM_SIGMOID
    if opts.get("half_split"):
        flags |= M3_FLAG_HALF_SPLIT
    return Shape(Bsz, T, H, P, N, R, int(chunk), io, flags, float(eps), int(nr or 0))


def _rotated(s: Shape) -> int:
    return s.rope_pairs if s.flags & M3_FLAG_PARTIAL_ROPE else s.dstate // 2


def _y_shape(s: Shape, mimo, mimo_o=None):
    """Shape of y: [B, T, H, P], with a trailing R for a MIMO call without mimo_o."""
    return (s.batch, s.seqlen, s.nheads, s.headdim) + ((s.rank,) if mimo and mimo_o is None else ())


def _inputs(s: Shape, x, B, C, dt, lam, theta, A, D, b_norm_w, c_norm_w, b_bias, c_bias, mimo,
            dt_bias=None, z=None, mimo_x=None, mimo_z=None, mimo_o=None, strided=True):
    """The C input block.  x, B, C, dt, lam, theta, a per-token A and z may be row-strided
    slices (see ``_need``) unless ``strided`` is False."""
    dev, io_t = x.device, x.dtype
    f32 = torch.float32
    bt = (s.batch, s.seqlen, s.nheads)
    bs = bt + (s.dstate,) + ((s.rank,) if mimo else ())
    rank_free = (s.batch, s.seqlen, s.nheads, s.headdim)
    full = rank_free + ((s.rank,) if mimo else ())
    proj = (s.nheads, s.rank, s.headdim)
    st = {}
    st["x"] = _need(x, "x", io_t, dev, rank_free if mimo_x is not None else full, rows=True)
    st["B"] = _need(B, "B", io_t, dev, bs, rows=True)
    st["C"] = _need(C, "C", io_t, dev, bs, rows=True)
    st["dt"] = _need(dt, "dt", f32, dev, bt, rows=True)
    st["lam"] = _need(lam, "lam", f32, dev, bt, rows=True)
    st["theta"] = _need(theta, "theta", f32, dev, bt + (_rotated(s),), rows=True)
    if s.flags & M3_FLAG_A_PER_TOKEN:
        st["A"] = _need(A, "A", f32, dev, bt, rows=True)
    else:
        _need(A, "A", f32, dev, (s.nheads,))
        st["A"] = 0
    _need(D, "D", f32, dev, (s.nheads,))
    _need(dt_bias, "dt_bias", f32, dev, (s.nheads,))
    st["z"] = _need(z, "z", io_t, dev, rank_free if mimo_z is not None else full, rows=True)
    _need(b_norm_w, "b_norm_w", f32, dev, (s.dstate,))
    _need(c_norm_w, "c_norm_w", f32, dev, (s.dstate,))
    _need(b_bias, "b_bias", f32, dev, (s.nheads, s.rank, s.dstate))
    _need(c_bias, "c_bias", f32, dev, (s.nheads, s.rank, s.dstate))
    for t, name in ((mimo_x, "mimo_x"), (mimo_z, "mimo_z"), (mimo_o, "mimo_o")):
        _need(t, name, f32, dev, proj)
    if not strided and any(v != 0 for v in st.values()):
        raise ValueError("this call takes contiguous inputs")
    return _Inputs(*(_ptr(t) for t in (x, B, C, dt, lam, theta, A, D, b_norm_w, c_norm_w,
                                        b_bias, c_bias, dt_bias, z, mimo_x, mimo_z, mimo_o)),
                   *(int(st[k]) for k in _ROW_STRIDED))


def new_state(batch, nheads, headdim, dstate, rank=1, device="cuda", rope_pairs=None):
    """Zero carried state (h, prev_B, prev_x, angle) as float32 device tensors.

    ``angle`` holds ``rope_pairs`` angles per (batch, head) (default N/2)."""
    z = lambda *sh: torch.zeros(sh, dtype=torch.float32, device=device)
    nr = dstate // 2 if rope_pairs is None else rope_pairs
    return dict(h=z(batch, nheads, dstate, headdim), prev_B=z(batch, nheads, dstate, rank),
                prev_x=z(batch, nheads, headdim, rank), angle=z(batch, nheads, nr))


def _state(s: Shape, st, dev, name):
    if st is None:
        return None
    _need(st["h"], f"{name}.h", torch.float32, dev, (s.batch, s.nheads, s.dstate, s.headdim))
    _need(st["prev_B"], f"{name}.prev_B", torch.float32, dev, (s.batch, s.nheads, s.dstate, s.rank))
    _need(st["prev_x"], f"{name}.prev_x", torch.float32, dev, (s.batch, s.nheads, s.headdim, s.rank))
    _need(st["angle"], f"{name}.angle", torch.float32, dev, (s.batch, s.nheads, _rotated(s)))
    return _State(*(_ptr(st[k]) for k in ("h", "prev_B", "prev_x", "angle")))


def m3_scan_workspace_bytes(shape: Shape) -> int:
    return int(load().m3_scan_workspace_bytes(ctypes.byref(shape)))


def _scan(mimo, x, B, C, dt, lam, theta, A, D, *, chunk=64, bcnorm=True, eps=1e-5,
          b_norm_w=None, c_norm_w=None, b_bias=None, c_bias=None, init=None, final=None,
          y=None, workspace=None, stream=None, rope_pairs=None, dt_softplus=False, dt_bias=None,
          lam_sigmoid=False, z=None, half_split=False, mimo_x=None, mimo_z=None, mimo_o=None):
    lib = load()
    s = _shape_of(x, B, chunk, bcnorm, eps, mimo, dict(rope_pairs=rope_pairs, A=A, dt_softplus=dt_softplus,
                                                        lam_sigmoid=lam_sigmoid, half_split=half_split,
                                                        mimo_x=mimo_x))
    inp = _inputs(s, x, B, C, dt, lam, theta, A, D, b_norm_w, c_norm_w, b_bias, c_bias, mimo,
                  dt_bias, z, mimo_x, mimo_z, mimo_o)
    ys = _y_shape(s, mimo, mimo_o)
    with _alloc_on(stream):
        if y is None:
            y = torch.empty(ys, dtype=x.dtype, device=x.device)
        else:
            _need(y, "y", x.dtype, x.device, ys)
        if final is True:
            final = new_state(s.batch, s.nheads, s.headdim, s.dstate, s.rank, x.device, _rotated(s))
        st_in = _state(s, init, x.device, "init")
        st_out = _state(s, final, x.device, "final")
        need = int(lib.m3_scan_workspace_bytes(ctypes.byref(s)))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
        _need(workspace, "workspace", torch.uint8, x.device)
        f = lib.m3_scan_mimo if mimo else lib.m3_scan_siso
        rc = f(ctypes.byref(s), ctypes.byref(inp), _ptr(y),
               ctypes.byref(st_in) if st_in is not None else None,
               ctypes.byref(st_out) if st_out is not None else None,
               _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream))
    _check(rc, "m3_scan_mimo" if mimo else "m3_scan_siso")
    return (y, final) if final is not None else y


def m3_scan_noalloc(x, B, C, dt, lam, theta, A, D, *, y, chunk=64, bcnorm=True, eps=1e-5,
                    b_norm_w=None, c_norm_w=None, b_bias=None, c_bias=None, init=None, final=None,
                    stream=None, rope_pairs=None, dt_softplus=False, dt_bias=None, lam_sigmoid=False,
                    z=None, half_split=False, mimo_x=None, mimo_z=None, mimo_o=None):
    """The allocation-free scan (any rank: B [B,T,H,N] is rank 1, [B,T,H,N,R] rank R) with the
    library's static scratch as workspace.  The caller passes the output ``y`` and, to get the
    final state, ``final`` (a state dict as from ``new_state``); nothing is allocated here or
    in the library, so the call may run under HIP graph capture."""
    lib = load()
    mimo = B.dim() == 5
    s = _shape_of(x, B, chunk, bcnorm, eps, mimo, dict(rope_pairs=rope_pairs, A=A, dt_softplus=dt_softplus,
                                                        lam_sigmoid=lam_sigmoid, half_split=half_split,
                                                        mimo_x=mimo_x))
    inp = _inputs(s, x, B, C, dt, lam, theta, A, D, b_norm_w, c_norm_w, b_bias, c_bias, mimo, dt_bias, z,
                  mimo_x, mimo_z, mimo_o)
    _need(y, "y", x.dtype, x.device, _y_shape(s, mimo, mimo_o))
    st_in = _state(s, init, x.device, "init")
    st_out = _state(s, final, x.device, "final")
    rc = lib.m3_scan_noalloc(ctypes.byref(s), ctypes.byref(inp), _ptr(y),
                             ctypes.byref(st_in) if st_in is not None else None,
                             ctypes.byref(st_out) if st_out is not None else None, _stream(stream))
    if rc == 3:
        need = int(lib.m3_scan_workspace_bytes(ctypes.byref(s)))
        raise RuntimeError(f"m3_scan_noalloc: this shape needs {need} bytes of workspace, more than the "
                           f"library's static scratch ({M3_STATIC_SCRATCH_BYTES} bytes); use m3_scan_mimo "
                           "with a workspace")
    _check(rc, "m3_scan_noalloc")
    return (y, final) if final is not None else y


def m3_scan_siso(x, B, C, dt, lam, theta, A, D, **kw):
    """SISO chunked scan.  x [B,T,H,P], B/C [B,T,H,N] (float32 or bfloat16); dt/lam [B,T,H],
    theta [B,T,H,N/2], A/D [H] float32.  ``final=True`` returns (y, final_state).

    Canonical-block options: ``rope_pairs`` (rotate only the leading pairs; theta and the
    state angle then hold that many), A of shape [B,T,H] (per-token decay rate),
    ``dt_softplus`` / ``dt_bias`` and ``lam_sigmoid`` (raw dt / lam), ``z`` (silu gate),
    ``half_split`` (rotation pairs (i, i + N/2))."""
    return _scan(False, x, B, C, dt, lam, theta, A, D, **kw)


def m3_scan_mimo(x, B, C, dt, lam, theta, A, D, **kw):
    """Rank-R MIMO chunked scan.  x [B,T,H,P,R], B/C [B,T,H,N,R]; ``chunk`` counts tokens.

    MIMO projections by learned per-rank vectors [H, R, P] (float32): ``mimo_x`` (x is then
    [B,T,H,P] and rank r reads x * mimo_x[:, r]), ``mimo_z`` (z is [B,T,H,P], expanded the same
    way) and ``mimo_o`` (y is [B,T,H,P] = sum_r mimo_o[:, r] * y_r).  x, B, C, dt, lam, theta,
    a per-token A and z may be row-strided slices of a wider buffer (e.g. the block's in_proj
    output): each token's row contiguous, rows evenly spaced."""
    return _scan(True, x, B, C, dt, lam, theta, A, D, **kw)


def m3_step(x, B, C, dt, lam, theta, A, D, state, *, bcnorm=True, eps=1e-5, b_norm_w=None,
            c_norm_w=None, b_bias=None, c_bias=None, y=None, stream=None, rope_pairs=None,
            dt_softplus=False, dt_bias=None, lam_sigmoid=False, z=None, half_split=False,
            mimo_x=None, mimo_z=None, mimo_o=None):
    """One decode step (T == 1) that updates ``state`` in place; returns y.

    x [B,1,H,P] (or [B,1,H,P,R]), B/C [B,1,H,N(,R)], dt/lam [B,1,H], theta [B,1,H,N/2]
    (the same options as the scans, MIMO projections and row-strided inputs included; a
    per-token A is [B,1,H])."""
    lib = load()
    mimo = B.dim() == 5
    s = _shape_of(x, B, 16, bcnorm, eps, mimo, dict(rope_pairs=rope_pairs, A=A, dt_softplus=dt_softplus,
                                                     lam_sigmoid=lam_sigmoid, half_split=half_split,
                                                     mimo_x=mimo_x))
    if s.seqlen != 1:
        raise ValueError("m3_step takes exactly one token (T == 1)")
    inp = _inputs(s, x, B, C, dt, lam, theta, A, D, b_norm_w, c_norm_w, b_bias, c_bias, mimo,
                  dt_bias, z, mimo_x, mimo_z, mimo_o)
    ys = _y_shape(s, mimo, mimo_o)
    with _alloc_on(stream):
        if y is None:
            y = torch.empty(ys, dtype=x.dtype, device=x.device)
        else:
            _need(y, "y", x.dtype, x.device, ys)
    st = _state(s, state, x.device, "state")
    rc = lib.m3_step(ctypes.byref(s), ctypes.byref(inp), _ptr(y), ctypes.byref(st), _stream(stream))
    _check(rc, "m3_step")
    return y


def m3_scan_bwd_workspace_bytes(shape: Shape) -> int:
    return int(load().m3_scan_bwd_workspace_bytes(ctypes.byref(shape)))


def m3_scan_bwd(x, B, C, dt, lam, theta, A, D, dy, *, bcnorm=True, eps=1e-5, b_norm_w=None,
                c_norm_w=None, b_bias=None, c_bias=None, init=None, dfinal=None, rope_pairs=None,
                dt_softplus=False, dt_bias=None, lam_sigmoid=False, z=None, workspace=None,
                stream=None, half_split=False, init_grad=True):
    """Gradients of m3_scan_siso / m3_scan_mimo (SISO when x is 4-D) given ``dy``.

    ``init`` is the forward call's initial state and ``dfinal`` the gradients of its final
    state (dicts h, prev_B, prev_x, angle; either may be None).  Returns a dict of tensors
    shaped like the inputs: x, B, C, dt, lam, theta, A, D, b_norm_w, c_norm_w, b_bias
    ([H, R, N]), c_bias, dt_bias, z (gated calls) and init (a dict of the initial state's
    gradients, or None with ``init_grad=False``, which also skips their kernel when no initial
    state is given).  Parameter gradients are sums over batch and tokens.
    """
    lib = load()
    mimo = x.dim() == 5
    s = _shape_of(x, B, 16, bcnorm, eps, mimo, dict(rope_pairs=rope_pairs, A=A, dt_softplus=dt_softplus,
                                                     lam_sigmoid=lam_sigmoid, half_split=half_split))
    inp = _inputs(s, x, B, C, dt, lam, theta, A, D, b_norm_w, c_norm_w, b_bias, c_bias, mimo,
                  dt_bias, z, strided=False)
    _need(dy, "dy", x.dtype, x.device, tuple(x.shape))
    dev, f32 = x.device, torch.float32
    H, N, R = s.nheads, s.dstate, s.rank
    with _alloc_on(stream):
        return _bwd_call(lib, s, inp, x, B, C, dt, lam, theta, A, D, dy, z, init, dfinal, workspace, stream,
                         dev, f32, H, N, R, init_grad)


def _bwd_call(lib, s, inp, x, B, C, dt, lam, theta, A, D, dy, z, init, dfinal, workspace, stream, dev, f32,
              H, N, R, init_grad=True):
    g = dict(x=torch.empty_like(x), B=torch.empty_like(B), C=torch.empty_like(C),
             dt=torch.empty_like(dt), lam=torch.empty_like(lam), theta=torch.empty_like(theta),
             A=torch.empty_like(A), D=torch.empty_like(D),
             b_norm_w=torch.empty(N, dtype=f32, device=dev), c_norm_w=torch.empty(N, dtype=f32, device=dev),
             b_bias=torch.empty((H, R, N), dtype=f32, device=dev),
             c_bias=torch.empty((H, R, N), dtype=f32, device=dev),
             dt_bias=torch.empty(H, dtype=f32, device=dev),
             z=torch.empty_like(z) if z is not None else None)
    gr = _Grads(*(_ptr(g[k]) for k in ("x", "B", "C", "dt", "lam", "theta", "A", "D", "b_norm_w",
                                         "c_norm_w", "b_bias", "c_bias", "dt_bias", "z")))
    st_in = _state(s, init, dev, "init")
    st_df = _state(s, dfinal, dev, "dfinal")
    dinit = new_state(s.batch, s.nheads, s.headdim, s.dstate, s.rank, dev, _rotated(s)) if init_grad else None
    st_di = _state(s, dinit, dev, "dinit")
    need = int(lib.m3_scan_bwd_workspace_bytes(ctypes.byref(s)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    rc = lib.m3_scan_bwd(ctypes.byref(s), ctypes.byref(inp), _ptr(dy),
                         ctypes.byref(st_in) if st_in is not None else None,
                         ctypes.byref(st_df) if st_df is not None else None,
                         ctypes.byref(gr), ctypes.byref(st_di) if st_di is not None else None, _ptr(workspace),
                         ctypes.c_size_t(workspace.numel()), _stream(stream))
    _check(rc, "m3_scan_bwd")
    g["init"] = dinit
    return g
