"""fp64 CPU oracle of the Mamba-3 trapezoidal selective scan.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
bench's CPU-baseline leg, never by the library.  It shares no code with the
HIP path.  The arithmetic lives in ``m3_oracle.c`` (plain C, double
precision, one sequential token loop per (batch, head)); this module only
marshals numpy arrays into it.  See the header of ``m3_oracle.c`` for what is
computed and which passage of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "m3_oracle_bwd.c"), os.path.join(_HERE, "m3_oracle.h")]
_LIB = os.path.join(_HERE, "_m3_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)


class _Args(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
        ("dstate", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("bcnorm", ctypes.c_int32), ("eps", ctypes.c_double),
        ("x", _dp), ("Bm", _dp), ("Cm", _dp), ("dt", _dp), ("lam", _dp), ("theta", _dp),
        ("A", _dp), ("D", _dp),
        ("b_norm_w", _dp), ("c_norm_w", _dp), ("b_bias", _dp), ("c_bias", _dp),
        ("h0", _dp), ("pB0", _dp), ("px0", _dp), ("ang0", _dp),
        ("y", _dp), ("h1", _dp), ("pB1", _dp), ("px1", _dp), ("ang1", _dp),
        ("mutation", ctypes.c_int32), ("nthreads", ctypes.c_int32),
        ("rope_pairs", ctypes.c_int32), ("a_per_token", ctypes.c_int32),
        ("dt_softplus", ctypes.c_int32), ("lam_sigmoid", ctypes.c_int32),
        ("dt_bias", _dp), ("z", _dp), ("half_split", ctypes.c_int32),
        ("mimo_x", _dp), ("mimo_z", _dp), ("mimo_o", _dp),
    ]


class _BwdArgs(ctypes.Structure):
    _fields_ = [
        ("f", ctypes.POINTER(_Args)),
        ("dy", _dp), ("dh1", _dp), ("dpB1", _dp), ("dpx1", _dp), ("dang1", _dp),
        ("dx", _dp), ("dB", _dp), ("dC", _dp), ("ddt", _dp), ("dlam", _dp), ("dtheta", _dp),
        ("dA", _dp), ("dz", _dp),
        ("dD", _dp), ("dbnw", _dp), ("dcnw", _dp), ("dbb", _dp), ("dcb", _dp), ("ddtb", _dp),
        ("dh0", _dp), ("dpB0", _dp), ("dpx0", _dp), ("dang0", _dp),
        ("mutation", ctypes.c_int32),
    ]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, -O2, no fast-math)."""
    newest = max(os.path.getmtime(f) for f in _SRCS)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", *[f for f in _SRCS if f.endswith(".c")], "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        # M3_ORACLE_LIB: an alternative build of the same sources (the sanitizer build of the
        # tests); the default is the in-tree -O2 build
        _lib = ctypes.CDLL(os.environ.get("M3_ORACLE_LIB") or build())
        _lib.m3o_scan.argtypes = [ctypes.POINTER(_Args)]
        _lib.m3o_scan.restype = ctypes.c_int
        _lib.m3o_scan_bwd.argtypes = [ctypes.POINTER(_BwdArgs)]
        _lib.m3o_scan_bwd.restype = ctypes.c_int
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(_dp) if a is not None else None


def scan(x, B, C, dt, lam, theta, A, D, *, bcnorm=True, eps=1e-5,
         b_norm_w=None, c_norm_w=None, b_bias=None, c_bias=None,
         init=None, nthreads=None, mutation=0, rope_pairs=None,
         dt_softplus=False, dt_bias=None, lam_sigmoid=False, z=None, half_split=False,
         mimo_x=None, mimo_z=None, mimo_o=None):
    """Run the sequential fp64 loop.

    Shapes: x [Bt,T,H,P] (or [Bt,T,H,P,R]), B/C [Bt,T,H,N] (or [...,N,R]),
    dt/lam [Bt,T,H], theta [Bt,T,H,NR], A [H] or [Bt,T,H] (a per-token decay
    rate, recognised by its shape), D [H]; optional gains [N] and biases
    [H,R,N]; ``init`` a dict with any of h [Bt,H,N,P], prev_B [Bt,H,N,R],
    prev_x [Bt,H,P,R], angle [Bt,H,NR].  NR = ``rope_pairs`` (default N/2:
    every pair rotates).  ``dt_softplus``/``dt_bias`` and ``lam_sigmoid``
    take dt and lam as raw values; ``z`` (shaped like x) gates the output
    with silu(z); ``half_split`` pairs components (i, i + N/2) instead of
    (2i, 2i + 1).

    MIMO projections by learned per-rank vectors, each [H, R, P]: ``mimo_x``
    (x is then rank-free [Bt,T,H,P] and the scan reads x * mimo_x[h, r]),
    ``mimo_z`` (z rank-free, the gate reads z * mimo_z[h, r]), ``mimo_o`` (y is
    the rank contraction sum_r mimo_o[h, r] * y_r, shaped [Bt,T,H,P]).

    Returns (y, final) with y shaped like x (the rank-expanded x with mimo_x,
    the contracted [Bt,T,H,P] with mimo_o; float64) and final a dict of float64
    arrays h, prev_B, prev_x, angle (angle is the unreduced running sum;
    prev_x holds the expanded x).
    """
    x = _f64(x)
    Bm, Cm = _f64(B), _f64(C)
    Bsz, T, H, P = x.shape[:4]
    R = Bm.shape[4] if Bm.ndim == 5 else 1
    if mimo_x is None and x.ndim == 5 and x.shape[4] != R:
        raise ValueError("oracle: x and B must have the same rank")
    N = Bm.shape[3]
    keep = [x, Bm, Cm]
    a = _Args()
    a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, a.rank = Bsz, T, H, P, N, R
    a.bcnorm, a.eps = int(bool(bcnorm)), float(eps)

    def put(name, arr):
        arr = _f64(arr)
        keep.append(arr)
        setattr(a, name, _ptr(arr))
        return arr

    a.x, a.Bm, a.Cm = _ptr(x), _ptr(Bm), _ptr(Cm)
    NR = N // 2 if rope_pairs is None else int(rope_pairs)
    a.rope_pairs = NR
    A = _f64(A)
    a.a_per_token = int(A.ndim == 3)
    if A.ndim == 3 and A.shape != (Bsz, T, H):
        raise ValueError("oracle: a per-token A must be [B, T, H]")
    a.dt_softplus, a.lam_sigmoid = int(bool(dt_softplus)), int(bool(lam_sigmoid))
    if NR > 0 and np.shape(theta)[-1] != NR:
        raise ValueError("oracle: theta must hold rope_pairs angles per token")
    yr_shape = (Bsz, T, H, P) + ((R,) if R > 1 or x.ndim == 5 else ())  # per-rank outputs
    zs = (Bsz, T, H, P) if mimo_z is not None else yr_shape
    if z is not None and np.shape(z) != zs:
        raise ValueError(f"oracle: z must be shaped {zs}")
    for name, arr in (("mimo_x", mimo_x), ("mimo_z", mimo_z), ("mimo_o", mimo_o)):
        if arr is not None and np.shape(arr) != (H, R, P):
            raise ValueError(f"oracle: {name} must be [H, R, P]")
    for name, arr in (("dt", dt), ("lam", lam), ("theta", theta if NR > 0 else None), ("A", A),
                      ("D", D), ("b_norm_w", b_norm_w), ("c_norm_w", c_norm_w),
                      ("b_bias", b_bias), ("c_bias", c_bias), ("dt_bias", dt_bias), ("z", z),
                      ("mimo_x", mimo_x), ("mimo_z", mimo_z), ("mimo_o", mimo_o)):
        put(name, arr)
    init = init or {}
    for name, key in (("h0", "h"), ("pB0", "prev_B"), ("px0", "prev_x"), ("ang0", "angle")):
        put(name, init.get(key))
    y = np.zeros((Bsz, T, H, P) if mimo_o is not None else yr_shape, dtype=np.float64)
    fin = dict(h=np.zeros((Bsz, H, N, P)), prev_B=np.zeros((Bsz, H, N, R)),
               prev_x=np.zeros((Bsz, H, P, R)), angle=np.zeros((Bsz, H, NR)))
    a.y = _ptr(y)
    a.h1, a.pB1, a.px1, a.ang1 = (_ptr(fin["h"]), _ptr(fin["prev_B"]),
                                  _ptr(fin["prev_x"]), _ptr(fin["angle"]))
    a.mutation = int(mutation)
    a.nthreads = int(nthreads or os.cpu_count() or 1)
    a.half_split = int(bool(half_split))
    rc = _load().m3o_scan(ctypes.byref(a))
    if rc != 0:
        raise ValueError("oracle: unsupported sizes")
    return y, fin


def _prepare(x, B, C, dt, lam, theta, A, D, bcnorm, eps, b_norm_w, c_norm_w, b_bias, c_bias, init,
             nthreads, mutation, rope_pairs, dt_softplus, dt_bias, lam_sigmoid, z):
    """The forward argument block (and the arrays it points into) for a call."""
    x = _f64(x)
    mimo = x.ndim == 5
    Bsz, T, H, P = x.shape[:4]
    R = x.shape[4] if mimo else 1
    Bm, Cm = _f64(B), _f64(C)
    N = Bm.shape[3]
    keep = [x, Bm, Cm]
    a = _Args()
    a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, a.rank = Bsz, T, H, P, N, R
    a.bcnorm, a.eps = int(bool(bcnorm)), float(eps)

    def put(name, arr):
        arr = _f64(arr)
        keep.append(arr)
        setattr(a, name, _ptr(arr))
        return arr

    a.x, a.Bm, a.Cm = _ptr(x), _ptr(Bm), _ptr(Cm)
    NR = N // 2 if rope_pairs is None else int(rope_pairs)
    a.rope_pairs = NR
    A = _f64(A)
    a.a_per_token = int(A.ndim == 3)
    a.dt_softplus, a.lam_sigmoid = int(bool(dt_softplus)), int(bool(lam_sigmoid))
    for name, arr in (("dt", dt), ("lam", lam), ("theta", theta if NR > 0 else None), ("A", A),
                      ("D", D), ("b_norm_w", b_norm_w), ("c_norm_w", c_norm_w),
                      ("b_bias", b_bias), ("c_bias", c_bias), ("dt_bias", dt_bias), ("z", z)):
        put(name, arr)
    init = init or {}
    for name, key in (("h0", "h"), ("pB0", "prev_B"), ("px0", "prev_x"), ("ang0", "angle")):
        put(name, init.get(key))
    a.mutation = int(mutation)
    a.nthreads = int(nthreads or os.cpu_count() or 1)
    return a, keep, (Bsz, T, H, P, N, R, NR)


def scan_bwd(x, B, C, dt, lam, theta, A, D, dy, *, bcnorm=True, eps=1e-5,
             b_norm_w=None, c_norm_w=None, b_bias=None, c_bias=None, init=None, dfinal=None,
             nthreads=None, mutation=0, rope_pairs=None, dt_softplus=False, dt_bias=None,
             lam_sigmoid=False, z=None, half_split=False):
    """Gradients of the scan by the fp64 reverse sweep (m3_oracle_bwd.c).

    Same inputs and options as ``scan``; ``dy`` is the gradient of y (shaped like x) and
    ``dfinal`` an optional dict of gradients of the final state (h, prev_B, prev_x, angle).
    Returns a dict of float64 gradients, each shaped like its input: x, B, C, dt, lam,
    theta, A (per head, or per token when A is), D, b_norm_w, c_norm_w, b_bias, c_bias
    ([H, R, N]), dt_bias, z (when gated), and init (a dict h, prev_B, prev_x, angle).
    Gradients of raw dt / lam when the activations are on.

    ``half_split``: the pairing (i, i + N/2) is the adjacent pairing on the N axis
    permuted (component c of pair i at 2i + c); the sweep runs on the permuted
    problem (B, C, gains, biases, the N rows of h and prev_B and of their final-state
    gradients) and the gradients of those inputs are permuted back.
    """
    if half_split:
        N = np.shape(B)[3]
        perm = np.concatenate([np.arange(0, N, 2), np.arange(1, N, 2)])  # user n -> adjacent slot
        fw = np.empty(N, dtype=np.int64)  # adjacent slot m holds user component fw[m]
        fw[perm] = np.arange(N)
        take = lambda v, ax: None if v is None else np.take(np.asarray(v, np.float64), fw, axis=ax)
        back = lambda v, ax: None if v is None else np.take(v, perm, axis=ax)
        st = lambda d: None if d is None else {k: (take(v, 2) if k in ("h", "prev_B") else v) for k, v in d.items()}
        g = scan_bwd(x, take(B, 3), take(C, 3), dt, lam, theta, A, D, dy, bcnorm=bcnorm, eps=eps,
                     b_norm_w=take(b_norm_w, 0), c_norm_w=take(c_norm_w, 0), b_bias=take(b_bias, 2),
                     c_bias=take(c_bias, 2), init=st(init), dfinal=st(dfinal), nthreads=nthreads,
                     mutation=mutation, rope_pairs=rope_pairs, dt_softplus=dt_softplus, dt_bias=dt_bias,
                     lam_sigmoid=lam_sigmoid, z=z)
        for k, ax in (("B", 3), ("C", 3), ("b_norm_w", 0), ("c_norm_w", 0), ("b_bias", 2), ("c_bias", 2)):
            g[k] = back(g[k], ax)
        for k in ("h", "prev_B"):
            g["init"][k] = back(g["init"][k], 2)
        return g
    a, keep, (Bsz, T, H, P, N, R, NR) = _prepare(
        x, B, C, dt, lam, theta, A, D, bcnorm, eps, b_norm_w, c_norm_w, b_bias, c_bias, init,
        nthreads, 0, rope_pairs, dt_softplus, dt_bias, lam_sigmoid, z)
    g = _BwdArgs()
    g.f = ctypes.pointer(a)
    dyv = _f64(dy)
    keep.append(dyv)
    g.dy = _ptr(dyv)
    dfinal = dfinal or {}
    for name, key in (("dh1", "h"), ("dpB1", "prev_B"), ("dpx1", "prev_x"), ("dang1", "angle")):
        arr = _f64(dfinal.get(key))
        keep.append(arr)
        setattr(g, name, _ptr(arr))
    xs = np.shape(x)
    out = dict(x=np.zeros(xs), B=np.zeros(np.shape(B)), C=np.zeros(np.shape(C)),
               dt=np.zeros((Bsz, T, H)), lam=np.zeros((Bsz, T, H)), theta=np.zeros((Bsz, T, H, NR)),
               A=np.zeros(np.shape(A)), D=np.zeros(H), b_norm_w=np.zeros(N), c_norm_w=np.zeros(N),
               b_bias=np.zeros((H, R, N)), c_bias=np.zeros((H, R, N)), dt_bias=np.zeros(H),
               z=np.zeros(xs) if z is not None else None)
    ini = dict(h=np.zeros((Bsz, H, N, P)), prev_B=np.zeros((Bsz, H, N, R)),
               prev_x=np.zeros((Bsz, H, P, R)), angle=np.zeros((Bsz, H, NR)))
    for name, key in (("dx", "x"), ("dB", "B"), ("dC", "C"), ("ddt", "dt"), ("dlam", "lam"),
                      ("dtheta", "theta"), ("dA", "A"), ("dz", "z"), ("dD", "D"), ("dbnw", "b_norm_w"),
                      ("dcnw", "c_norm_w"), ("dbb", "b_bias"), ("dcb", "c_bias"), ("ddtb", "dt_bias")):
        setattr(g, name, _ptr(out[key]))
    for name, key in (("dh0", "h"), ("dpB0", "prev_B"), ("dpx0", "prev_x"), ("dang0", "angle")):
        setattr(g, name, _ptr(ini[key]))
    g.mutation = int(mutation)
    rc = _load().m3o_scan_bwd(ctypes.byref(g))
    if rc != 0:
        raise ValueError("oracle: unsupported sizes")
    out["init"] = ini
    return out
