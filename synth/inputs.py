"""Seeded synthetic inputs for the Mamba-3 trapezoidal selective scan.

This module is shared by the fp64 oracle (test infrastructure) and the HIP
path's tests and bench.  It draws random numbers and rounds them to storage
precision; it holds none of the scan's arithmetic (no discretisation, no norm,
no rotation, no recurrence).

Recipe (one ``numpy.random.default_rng(seed)`` per workload, PCG64, draws in
this fixed order):

    x      ~ N(0, 1)                         [B, T, H, P]   (rank R: [B, T, H, P, R])
    dt     = softplus(N(0, 1) - dt_shift)    [B, T, H]      (dt_shift 4; 5 for the long case)
    A      = -exp(U(0, ln 16))               [H]
    lam    = sigmoid(N(0, 1))                [B, T, H]
    theta  ~ U(0, pi/8)                      [B, T, H, N/2]
    B, C   ~ N(0, 1) (raw, before the norm)  [B, T, H, N]   (rank R: [B, T, H, N, R])
    D      ~ N(0, 1)                         [H]

softplus / sigmoid are the input activations of the Mamba-3 block (dt and the
trapezoid gate lambda are handed to the scan already activated).  For bf16
workloads x, B and C are rounded to bfloat16 with round-to-nearest-even and
both sides read exactly those values; everything else is float32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int   # P
    dstate: int    # N
    rank: int      # R (1 = SISO)
    chunk: int     # Q tokens per chunk on the GPU path
    io: str        # "f32" or "bf16": dtype of x, B, C, y
    dt_shift: float = 4.0
    seed: int = 0
    steps: int = 0  # >0: decode workload (one token per step, `steps` steps)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# The five workloads.  Shapes follow the 434M-parameter Mamba-3-Lite layer
# (d_model 1024, 16 heads of 64, state 64) and the tiny debug layer.
WORKLOADS = {
    0: Workload("tiny_siso_f32", 1, 64, 2, 4, 4, 1, 16, "f32", 4.0, seed=0),
    1: Workload("siso_b4_t2048_h16_p64_n64_bf16", 4, 2048, 16, 64, 64, 1, 64, "bf16", 4.0, seed=1),
    2: Workload("mimo_r4_b4_t2048_h16_p64_n64_bf16", 4, 2048, 16, 64, 64, 4, 16, "bf16", 4.0, seed=2),
    3: Workload("siso_long_b1_t16384_h32_p64_n128_bf16", 1, 16384, 32, 64, 128, 1, 128, "bf16", 5.0, seed=3),
    4: Workload("step_b256_h16_p64_n64_bf16_x512", 256, 512, 16, 64, 64, 1, 64, "bf16", 4.0, seed=4, steps=512),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bfloat16 value (ties to even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    # NaN stays NaN (none are drawn, kept for completeness)
    return np.where(np.isnan(a), a, out).astype(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def _sigmoid(v: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-v))


def make_inputs(w: Workload, *, batch: int | None = None, seqlen: int | None = None,
                seed: int | None = None) -> dict:
    """Draw one workload's inputs.  Returns float32 numpy arrays.

    Keys: x, B, C, dt, lam, theta, A, D.  x/B/C are bf16-rounded when
    ``w.io == "bf16"``.  ``batch``/``seqlen``/``seed`` override the workload's.
    """
    Bsz = w.batch if batch is None else batch
    T = w.seqlen if seqlen is None else seqlen
    H, P, N, R = w.nheads, w.headdim, w.dstate, w.rank
    rng = np.random.default_rng(w.seed if seed is None else seed)
    xs = (Bsz, T, H, P) if R == 1 else (Bsz, T, H, P, R)
    bs = (Bsz, T, H, N) if R == 1 else (Bsz, T, H, N, R)
    x = rng.standard_normal(xs, dtype=np.float32)
    dt = _softplus(rng.standard_normal((Bsz, T, H)) - w.dt_shift).astype(np.float32)
    A = (-np.exp(rng.uniform(0.0, math.log(16.0), H))).astype(np.float32)
    lam = _sigmoid(rng.standard_normal((Bsz, T, H))).astype(np.float32)
    theta = rng.uniform(0.0, math.pi / 8, (Bsz, T, H, N // 2)).astype(np.float32)
    Bm = rng.standard_normal(bs, dtype=np.float32)
    Cm = rng.standard_normal(bs, dtype=np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    if w.io == "bf16":
        x, Bm, Cm = bf16_round(x), bf16_round(Bm), bf16_round(Cm)
    return dict(x=x, B=Bm, C=Cm, dt=dt, lam=lam, theta=theta, A=A, D=D)


def make_state(w: Workload, *, batch: int | None = None, seed: int = 1234,
               scale: float = 1.0, rope_pairs: int | None = None) -> dict:
    """A random carried state (h, prev_B, prev_x, angle) for streaming tests.

    ``angle`` holds ``rope_pairs`` angles per (batch, head) (default N/2)."""
    Bsz = w.batch if batch is None else batch
    H, P, N, R = w.nheads, w.headdim, w.dstate, w.rank
    rng = np.random.default_rng(seed)
    h = (scale * rng.standard_normal((Bsz, H, N, P))).astype(np.float32)
    pB = rng.standard_normal((Bsz, H, N, R)).astype(np.float32)
    px = rng.standard_normal((Bsz, H, P, R)).astype(np.float32)
    nr = N // 2 if rope_pairs is None else rope_pairs
    ang = rng.uniform(0.0, 2 * math.pi, (Bsz, H, nr)).astype(np.float32)
    return dict(h=h, prev_B=pB, prev_x=px, angle=ang)


def make_norm_params(w: Workload, *, seed: int = 77) -> dict:
    """Random norm gains [N] and per-(head, rank) biases [H, R, N]."""
    H, N, R = w.nheads, w.dstate, w.rank
    rng = np.random.default_rng(seed)
    return dict(
        b_norm_w=(1.0 + 0.1 * rng.standard_normal(N)).astype(np.float32),
        c_norm_w=(1.0 + 0.1 * rng.standard_normal(N)).astype(np.float32),
        b_bias=(0.1 * rng.standard_normal((H, R, N))).astype(np.float32),
        c_bias=(0.1 * rng.standard_normal((H, R, N))).astype(np.float32),
    )


def custom(name="custom", **kw) -> Workload:
    """A workload with explicit sizes (tests use it for ragged/edge shapes)."""
    base = dict(batch=1, seqlen=64, nheads=2, headdim=4, dstate=4, rank=1, chunk=16, io="f32")
    base.update(kw)
    return Workload(name, **base)


def make_block_inputs(w: Workload, *, rope_pairs: int | None = None, batch: int | None = None,
                      seqlen: int | None = None, seed: int | None = None) -> dict:
    """Inputs of the canonical-block options, drawn after ``make_inputs``' recipe.

    One more ``default_rng(seed + 7919)`` stream, in this order:

        dt_raw  = N(0, 1) - dt_shift          [B, T, H]   (the scan applies softplus(dt_raw + dt_bias))
        dt_bias ~ N(0, 0.25^2)                [H]
        lam_raw ~ N(0, 1)                     [B, T, H]   (the scan applies the sigmoid)
        A_tok   = -exp(U(0, ln 16))           [B, T, H]   per-token decay rate
        z       ~ N(0, 1)                     like x      (gate input; bf16-rounded for bf16 io)
        theta_p ~ U(0, pi/8)                  [B, T, H, rope_pairs]  (rope_pairs = N/4 by default)
    """
    Bsz = w.batch if batch is None else batch
    T = w.seqlen if seqlen is None else seqlen
    H, P, N, R = w.nheads, w.headdim, w.dstate, w.rank
    nr = N // 4 if rope_pairs is None else rope_pairs
    rng = np.random.default_rng((w.seed if seed is None else seed) + 7919)
    xs = (Bsz, T, H, P) if R == 1 else (Bsz, T, H, P, R)
    dt_raw = (rng.standard_normal((Bsz, T, H)) - w.dt_shift).astype(np.float32)
    dt_bias = (0.25 * rng.standard_normal(H)).astype(np.float32)
    lam_raw = rng.standard_normal((Bsz, T, H)).astype(np.float32)
    A_tok = (-np.exp(rng.uniform(0.0, math.log(16.0), (Bsz, T, H)))).astype(np.float32)
    z = rng.standard_normal(xs, dtype=np.float32)
    theta_p = rng.uniform(0.0, math.pi / 8, (Bsz, T, H, nr)).astype(np.float32)
    if w.io == "bf16":
        z = bf16_round(z)
    return dict(dt_raw=dt_raw, dt_bias=dt_bias, lam_raw=lam_raw, A_tok=A_tok, z=z, theta_p=theta_p)


def make_mimo_proj(w: Workload, *, batch: int | None = None, seqlen: int | None = None,
                   seed: int | None = None) -> dict:
    """Rank-free x and z and the MIMO projection vectors, drawn after ``make_inputs``' recipe.

    One more ``default_rng(seed + 104729)`` stream, in this order:

        x_free ~ N(0, 1)          [B, T, H, P]   (read as x_r = x_free * mimo_x[h, r])
        z_free ~ N(0, 1)          [B, T, H, P]   (read as z_r = z_free * mimo_z[h, r])
        mimo_x, mimo_z, mimo_o ~ U(-1.5, 1.5)   [H, R, P] each

    x_free and z_free are bf16-rounded for bf16 workloads; the vectors stay float32.
    """
    Bsz = w.batch if batch is None else batch
    T = w.seqlen if seqlen is None else seqlen
    H, P, R = w.nheads, w.headdim, w.rank
    rng = np.random.default_rng((w.seed if seed is None else seed) + 104729)
    x_free = rng.standard_normal((Bsz, T, H, P), dtype=np.float32)
    z_free = rng.standard_normal((Bsz, T, H, P), dtype=np.float32)
    vec = {k: rng.uniform(-1.5, 1.5, (H, R, P)).astype(np.float32) for k in ("mimo_x", "mimo_z", "mimo_o")}
    if w.io == "bf16":
        x_free, z_free = bf16_round(x_free), bf16_round(z_free)
    return dict(x_free=x_free, z_free=z_free, **vec)
