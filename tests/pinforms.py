"""Independent forms of the Mamba-3 scan that pin the fp64 oracle.

Test-only numpy code, written separately from the oracle's C loop (different
structure: matrices, complex numbers, closed forms, a chunked algorithm).
None of it is used by the HIP library.  Each form cites the passage of the
pages it restates.
"""
from __future__ import annotations

import numpy as np


def _as_mimo(x, B, C):
    """Give SISO arrays a unit rank axis."""
    if x.ndim == 4:
        return x[..., None], B[..., None], C[..., None], True
    return x, B, C, False


def prep_hat(V, gain, bias, h, bcnorm, eps):
    """RMSNorm over N (optional gain) then per-(head, rank) bias.

    V: [T, N, R] for one head.  dotLLM PR #136 "Key findings": bias after the
    norm, before the rotation; torchmamba "Math notes": BCNorm + bias.
    """
    V = V.astype(np.float64)
    if bcnorm:
        rms = np.sqrt(np.mean(V * V, axis=1, keepdims=True) + eps)
        V = V / rms
        if gain is not None:
            V = V * np.asarray(gain, np.float64)[None, :, None]
    if bias is not None:
        V = V + np.transpose(np.asarray(bias, np.float64)[h], (1, 0))[None]  # [H,R,N] -> [N,R]
    return V


def rotate(V, ang):
    """Rotate pairs (2i, 2i+1) of V [T, N, R] by angles ang [T, N/2] (standard direction)."""
    c, s = np.cos(ang)[..., None], np.sin(ang)[..., None]
    u, w = V[:, 0::2, :], V[:, 1::2, :]
    out = np.empty_like(V)
    out[:, 0::2, :] = u * c - w * s
    out[:, 1::2, :] = u * s + w * c
    return out


def quadratic(x, B, C, dt, lam, theta, A, D, *, bcnorm=True, eps=1e-5,
              gains=(None, None), biases=(None, None)):
    """Parallel (quadratic) form  Y = (L o C~B~^T) X + D X  with  L = S(alpha) @ Band.

    torchmamba "Math notes" (M3 SISO): the parallel mask is the 1-semiseparable
    decay matrix times a bidiagonal band (a matrix product, not Hadamard);
    "API reference": the quadratic oracle is only for short sequences.  Zero
    initial state.  For rank R the rows are (token, rank) pairs and the mask
    depends on tokens only.
    """
    x, B, C, siso = _as_mimo(x, B, C)
    Bsz, T, H, P, R = x.shape
    N = B.shape[3]
    assert T <= 16, "quadratic form is for short sequences"
    y = np.zeros((Bsz, T, H, P, R))
    for b in range(Bsz):
        for h in range(H):
            ang = np.zeros((T, N // 2))
            NR = np.shape(theta)[-1]  # rotated pairs: the leading NR (all N/2 by default)
            ang[:, :NR] = np.cumsum(np.asarray(theta, np.float64)[b, :, h, :], axis=0)  # inclusive
            Bt = rotate(prep_hat(B[b, :, h], gains[0], biases[0], h, bcnorm, eps), ang)
            Ct = rotate(prep_hat(C[b, :, h], gains[1], biases[1], h, bcnorm, eps), ang)
            d = dt[b, :, h].astype(np.float64)
            la = lam[b, :, h].astype(np.float64)
            Ah = np.asarray(A, np.float64)
            al = np.exp(d * (Ah[b, :, h] if Ah.ndim == 3 else Ah[h]))  # A per token or per head
            be = al * d * (1.0 - la)
            ga = la * d
            S = np.zeros((T, T))
            for t in range(T):
                for u in range(t + 1):
                    S[t, u] = np.prod(al[u + 1:t + 1])
            band = np.diag(ga)
            for s in range(T - 1):
                band[s + 1, s] = be[s + 1]
            L = S @ band
            # G[(t,r),(s,r')] = C~_t[:,r] . B~_s[:,r']
            G = np.einsum("tnr,snq->trsq", Ct, Bt)
            M = G * L[:, None, :, None]
            xt = x[b, :, h].astype(np.float64)  # [T, P, R]
            y[b, :, h] = np.einsum("trsq,spq->tpr", M, xt) + float(D[h]) * xt
    return y[..., 0] if siso else y


def complex_state_loop(x, B, C, dt, lam, theta, A, D, *, bcnorm=True, eps=1e-5,
                       gains=(None, None), biases=(None, None), half_split=False):
    """The scan with an explicitly complex state and no cumulative angle.

    torchmamba "Math notes" (M3 SISO, RoPE trick): the complex state
    transition is equivalent to accumulated rotations of B and C.  Here pair
    i of the state is one complex number and the per-step transition is
    alpha_t * exp(-i theta_t); B and C stay unrotated:
        g_t = exp(-i theta_t) (alpha_t g_{t-1} + beta_t B^_{t-1} x_{t-1}^T) + gamma_t B^_t x_t^T
        y_t = Re(conj(C^_t) . g_t)   (summed over pairs; real dot product of 2-vectors)
    Zero initial state.  ``half_split``: the complex number of pair i is made of
    components i and i + N/2 instead of 2i and 2i + 1.
    """
    x, B, C, siso = _as_mimo(x, B, C)
    Bsz, T, H, P, R = x.shape
    N = B.shape[3]
    y = np.zeros((Bsz, T, H, P, R))
    for b in range(Bsz):
        for h in range(H):
            Bh = prep_hat(B[b, :, h], gains[0], biases[0], h, bcnorm, eps)
            Ch = prep_hat(C[b, :, h], gains[1], biases[1], h, bcnorm, eps)
            if half_split:
                Bc = Bh[:, :N // 2, :] + 1j * Bh[:, N // 2:, :]
                Cc = Ch[:, :N // 2, :] + 1j * Ch[:, N // 2:, :]
            else:
                Bc = Bh[:, 0::2, :] + 1j * Bh[:, 1::2, :]   # [T, N/2, R]
                Cc = Ch[:, 0::2, :] + 1j * Ch[:, 1::2, :]
            g = np.zeros((N // 2, P), dtype=np.complex128)
            prev = np.zeros((N // 2, P), dtype=np.complex128)
            Ah = np.asarray(A, np.float64)
            NR = np.shape(theta)[-1]  # pairs past NR do not rotate
            for t in range(T):
                d = float(dt[b, t, h]); la = float(lam[b, t, h])
                al = np.exp(d * (Ah[b, t, h] if Ah.ndim == 3 else Ah[h]))
                be = al * d * (1.0 - la)
                ga = la * d
                xt = x[b, t, h].astype(np.float64)  # [P, R]
                cur = Bc[t] @ xt.T                    # sum_r B^[:,r] x[:,r]^T  -> [N/2, P]
                th = np.zeros(N // 2)
                th[:NR] = np.asarray(theta, np.float64)[b, t, h]
                rot = np.exp(-1j * th)[:, None]
                g = rot * (al * g + be * prev) + ga * cur
                prev = cur
                # real dot product of 2-vectors: Re(conj(c) * g)
                y[b, t, h] = np.real(np.conj(Cc[t]).T @ g).T + float(D[h]) * xt
    return y[..., 0] if siso else y


def mamba2_loop(x, B, C, dt, A, D, *, bcnorm=False, eps=1e-5):
    """Mamba-2 scalar-decay recurrence  h = exp(dt A) h + dt B x^T,  y = C^T h + D x.

    torchmamba "Models" (Mamba-2 row) and the reduction paragraph (M2 -> Mamba-3
    SISO at lambda = 1, theta = 0).  SISO only, zero initial state.
    """
    x = np.asarray(x, np.float64)
    Bsz, T, H, P = x.shape
    N = B.shape[3]
    y = np.zeros((Bsz, T, H, P))
    for b in range(Bsz):
        for h in range(H):
            Bh = prep_hat(B[b, :, h][..., None], None, None, h, bcnorm, eps)[..., 0]
            Ch = prep_hat(C[b, :, h][..., None], None, None, h, bcnorm, eps)[..., 0]
            st = np.zeros((N, P))
            for t in range(T):
                a = np.exp(float(dt[b, t, h]) * float(A[h]))
                st = a * st + float(dt[b, t, h]) * np.outer(Bh[t], x[b, t, h])
                y[b, t, h] = Ch[t] @ st + float(D[h]) * x[b, t, h]
    return y


def mamba2_quadratic(x, B, C, dt, A, D):
    """Mamba-2 dual form  Y = (L o C B^T)(dt * X) + D X,  L[t,s] = exp(sum_{s<k<=t} dt_k A).

    torchmamba "Math notes" (M2: M = L o (C B^T), quadratic dual).  SISO, no norm.
    """
    x = np.asarray(x, np.float64)
    Bsz, T, H, P = x.shape
    y = np.zeros((Bsz, T, H, P))
    for b in range(Bsz):
        for h in range(H):
            la = dt[b, :, h].astype(np.float64) * float(A[h])
            cs = np.cumsum(la)
            L = np.tril(np.exp(cs[:, None] - cs[None, :]))
            G = C[b, :, h].astype(np.float64) @ B[b, :, h].astype(np.float64).T
            xd = x[b, :, h].astype(np.float64) * dt[b, :, h].astype(np.float64)[:, None]
            y[b, :, h] = (L * G) @ xd + float(D[h]) * x[b, :, h]
    return y


def closed_form(T, N, dt, A, lam, theta, eps=None):
    """Exact output for constant dt, lambda, theta, B = C = 1 (all N), x = 1 (P = R = 1), D = 0.

    Derived from the recurrence (torchmamba "Models", M3 SISO row) with
    alpha = exp(dt A), beta = alpha dt (1-lambda), gamma = lambda dt: with
    z = exp(dt A) exp(-i theta),
        y_t = N * Re[ gamma (1 - z^{t+1})/(1 - z) + dt (1-lambda) (z - z^{t+1})/(1 - z) ].
    With the norm on, B^ = C^ = 1/sqrt(1 + eps), so y scales by 1/(1 + eps).
    """
    z = np.exp(dt * A) * np.exp(-1j * theta)
    ga = lam * dt
    t = np.arange(T)
    y = N * np.real(ga * (1 - z ** (t + 1)) / (1 - z) + dt * (1 - lam) * (z - z ** (t + 1)) / (1 - z))
    if eps is not None:
        y = y / (1.0 + eps)
    return y


def _round_bf16(a):
    a = np.asarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def chunked(x, B, C, dt, lam, theta, A, D, Q, *, bcnorm=True, eps=1e-5,
            gains=(None, None), biases=(None, None), init=None, bf16_ops=False):
    """Chunkwise form with a shifted state and chunk-local rotation frames.

    This is the algorithm the GPU path uses, written on the CPU to check it
    against the sequential loop (and, with ``bf16_ops``, to predict the error
    of bf16 matrix-core operands).  Sources:
      - torchmamba "Math notes" (M2): chunkwise SSD = intra-chunk quadratic
        part plus a factored inter-chunk state carry.
      - dotLLM PR #136 "Mamba-3 streaming decode": the trapezoid's two SSDs
        fold into one SSD whose per-token scale is gamma_t + eta_t with
        eta_t = dt_{t+1}(1 - lambda_{t+1}) (a one-token lookahead that must
        cross chunk edges), and the carried boundary term
        dt_0 (1 - lambda_0) k_state v_state is added to the state first.
    Shifted state h'_t = h_t + eta_t B~_t x_t^T obeys
        h'_t = alpha_t h'_{t-1} + (gamma_t + eta_t) B~_t x_t^T,
        y_t  = C~_t^T h'_t - eta_t (C~_t . B~_t) x_t + D x_t,
    with eta = 0 after the last token of the call.
    """
    x, B, C, siso = _as_mimo(x, B, C)
    Bsz, T, H, P, R = x.shape
    N = B.shape[3]
    N2 = N // 2
    rnd = _round_bf16 if bf16_ops else (lambda v: v)
    y = np.zeros((Bsz, T, H, P, R))
    fin = dict(h=np.zeros((Bsz, H, N, P)), prev_B=np.zeros((Bsz, H, N, R)),
               prev_x=np.zeros((Bsz, H, P, R)), angle=np.zeros((Bsz, H, N2)))
    init = init or {}

    def rot_state(S, ang):  # rotate rows (2i, 2i+1) of S [N, P] by ang [N/2]
        c, s = np.cos(ang)[:, None], np.sin(ang)[:, None]
        out = np.empty_like(S)
        out[0::2] = S[0::2] * c - S[1::2] * s
        out[1::2] = S[0::2] * s + S[1::2] * c
        return out

    for b in range(Bsz):
        for h in range(H):
            d = dt[b, :, h].astype(np.float64)
            la = lam[b, :, h].astype(np.float64)
            logal = d * float(A[h])
            ga = la * d
            eta = np.zeros(T)
            eta[:-1] = d[1:] * (1.0 - la[1:])
            scale = ga + eta
            Bh = prep_hat(B[b, :, h], gains[0], biases[0], h, bcnorm, eps)
            Ch = prep_hat(C[b, :, h], gains[1], biases[1], h, bcnorm, eps)
            xt = x[b, :, h].astype(np.float64)
            th = theta[b, :, h].astype(np.float64)
            base = np.array(init["angle"][b, h], np.float64) if "angle" in init else np.zeros(N2)
            Hs = np.array(init["h"][b, h], np.float64) if "h" in init else np.zeros((N, P))
            if "prev_B" in init and T > 0:
                eta_m1 = d[0] * (1.0 - la[0])
                Hs = Hs + eta_m1 * np.asarray(init["prev_B"][b, h], np.float64) @ \
                    np.asarray(init["prev_x"][b, h], np.float64).T
            Hs = rot_state(Hs, -base)  # into the local frame of chunk 0
            for c0 in range(0, T, Q):
                c1 = min(T, c0 + Q)
                n = c1 - c0
                phi = np.cumsum(th[c0:c1], axis=0)        # inclusive, chunk-local
                Bt = rnd(rotate(Bh[c0:c1], phi))           # [n, N, R]
                Ct = rnd(rotate(Ch[c0:c1], phi))
                cs = np.cumsum(logal[c0:c1])
                Lm = np.zeros((n, n))
                for t in range(n):
                    for s in range(t):
                        Lm[t, s] = np.exp(cs[t] - cs[s]) * scale[c0 + s]
                    Lm[t, t] = ga[c0 + t]
                G = np.einsum("tnr,snq->trsq", Ct, Bt)
                M = rnd(G * Lm[:, None, :, None])
                Yi = np.einsum("trsq,spq->tpr", M, xt[c0:c1])
                Hb = rnd(Hs)
                Yo = np.einsum("tnr,np->tpr", Ct, Hb) * np.exp(cs)[:, None, None]
                y[b, c0:c1, h] = Yi + Yo + float(D[h]) * xt[c0:c1]
                w = np.exp(cs[-1] - cs) * scale[c0:c1]    # [n]
                Bw = rnd(Bt * w[:, None, None])
                S = np.einsum("snq,spq->np", Bw, xt[c0:c1])
                Hs = rot_state(np.exp(cs[-1]) * Hs + S, -phi[-1])
                base = base + phi[-1]
            fin["h"][b, h] = rot_state(Hs, base)
            fin["angle"][b, h] = base
            if T > 0:
                fin["prev_B"][b, h] = rotate(Bh[T - 1:T], base[None])[0]
                fin["prev_x"][b, h] = xt[T - 1]
            else:
                for k in ("prev_B", "prev_x"):
                    if k in init:
                        fin[k][b, h] = init[k][b, h]
    if siso:
        y = y[..., 0]
    return y, fin
