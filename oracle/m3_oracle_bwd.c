/*
 * m3_oracle_bwd.c -- plain fp64 CPU gradients of the Mamba-3 trapezoidal
 * selective scan computed by m3_oracle.c.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this.  It shares no code with the HIP
 * library.  The gradients are pinned by central finite differences of the
 * forward oracle (tests/test_oracle_bwd_pins.py).
 *
 * The pages ask for gradients of the scan (torchmamba "Verification": fp64
 * gradchecks of the scans; dotLLM PR #136: the block is a training
 * component).  They print no backward algorithm; this file is reverse-mode
 * differentiation of the forward loop written out by hand, in reverse token
 * order, one (batch, head) sequence at a time:
 *
 *   forward (stored for every token): Theta_t, the normalised / biased B^, C^
 *   and their norm factors, the rotated B~, C~, alpha, beta, gamma, the
 *   activated dt and lambda, the state h_t, the ungated output.
 *
 *   reverse, with hb the gradient of the state h_t (hb_T = upstream final h):
 *     gate:      zb = yb * yfull * silu'(z),   yb <- yb * silu(z)
 *     skip:      Db += yb . x,   xb_t += D yb_t
 *     output:    hb_t += sum_r C~_{t,r} yb_{t,r}^T,   C~b_{t,r} = h_t yb_{t,r}
 *     update:    h_t = alpha_t h_{t-1} + beta_t sum_r B~_{t-1,r} x_{t-1,r}^T + gamma_t sum_r B~_{t,r} x_{t,r}^T
 *                B~b_{t,r} += gamma_t hb_t x_{t,r},    xb_{t,r} += gamma_t hb_t^T B~_{t,r}
 *                B~b_{t-1,r} += beta_t hb_t x_{t-1,r}, xb_{t-1,r} += beta_t hb_t^T B~_{t-1,r}
 *                gammab = sum_r B~_{t,r}^T hb_t x_{t,r},  betab = sum_r B~_{t-1,r}^T hb_t x_{t-1,r},
 *                alphab = <hb_t, h_{t-1}>,   hb_{t-1} = alpha_t hb_t
 *     scalars:   alpha = exp(dt A), beta = alpha dt (1 - lambda), gamma = lambda dt
 *     rotation:  B^b = Rot(-Theta) B~b;  Thetab_i += u v~b... (the 2-D cross product of a
 *                rotated pair with its gradient);  thetab_t = sum_{k >= t} Thetab_k
 *     norm:      B^ = g B r + bias, r = (mean B^2 + eps)^(-1/2)
 *   The carried initial state (h, prev_B, prev_x, angle) receives the
 *   gradients of h_{-1}, B~_{-1}, x_{-1} and Theta_{-1}.
 *
 * Layouts are those of m3_oracle.c; every gradient has the shape of its
 * input.  Parameter gradients (A per head, D, gains, biases, dt bias) are
 * sums over batch and tokens.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "m3_oracle.h"

typedef struct {
    const m3o_args *f;  /* forward inputs and options (its output pointers are ignored) */
    /* upstream gradients */
    const double *dy;                          /* like y */
    const double *dh1, *dpB1, *dpx1, *dang1;  /* final state, or NULL (= 0) */
    /* gradients (NULL = not wanted) */
    double *dx, *dB, *dC, *ddt, *dlam, *dtheta, *dA, *dz;
    double *dD, *dbnw, *dcnw, *dbb, *dcb, *ddtb;
    double *dh0, *dpB0, *dpx0, *dang0;
    int32_t mutation; /* planted mistakes for the pin tests; 0 in real use */
} m3o_bwd_args;

static double sp(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }
static double sg(double v) { return 1.0 / (1.0 + exp(-v)); }

/* per-sequence partial sums of the parameter gradients */
typedef struct {
    double *dA, *dD, *dbnw, *dcnw, *dbb, *dcb, *ddtb; /* dA per head only when A is per head */
} partial_t;

static void bwd_sequence(const m3o_bwd_args *g, int64_t b, int h, partial_t *pp) {
    const m3o_args *a = g->f;
    const int64_t T = a->seqlen;
    const int H = a->nheads, P = a->headdim, N = a->dstate, R = a->rank, N2 = N / 2, NR = a->rope_pairs;
    const int64_t bh = b * H + h;
    /* ---- forward, storing what the reverse sweep reads */
    double *hs = calloc((size_t)(T + 1) * N * P, sizeof(double));   /* h_{t-1} at t = 0 .. h_{T-1} */
    double *Bt = calloc((size_t)(T + 1) * N * R, sizeof(double));   /* B~_{t-1}, t = 0 .. T */
    double *Ct = calloc((size_t)(T > 0 ? T : 1) * N * R, sizeof(double));
    double *Bh = calloc((size_t)(T > 0 ? T : 1) * N * R, sizeof(double)); /* B^ (before the rotation) */
    double *Ch = calloc((size_t)(T > 0 ? T : 1) * N * R, sizeof(double));
    double *rb = calloc((size_t)(T > 0 ? T : 1) * R, sizeof(double)), *rc = calloc((size_t)(T > 0 ? T : 1) * R, sizeof(double));
    double *Th = calloc((size_t)(T + 1) * (N2 > 0 ? N2 : 1), sizeof(double)); /* Theta_{t-1}, t = 0 .. T */
    double *al = calloc((size_t)(T > 0 ? T : 1), sizeof(double)), *be = calloc((size_t)(T > 0 ? T : 1), sizeof(double));
    double *ga = calloc((size_t)(T > 0 ? T : 1), sizeof(double)), *dtv = calloc((size_t)(T > 0 ? T : 1), sizeof(double));
    double *lmv = calloc((size_t)(T > 0 ? T : 1), sizeof(double)), *Av = calloc((size_t)(T > 0 ? T : 1), sizeof(double));
    double *yf = calloc((size_t)(T > 0 ? T : 1) * P * R, sizeof(double)); /* ungated output */
    double *xp = calloc((size_t)P * R, sizeof(double));                  /* x_{-1} */
    if (a->h0) memcpy(hs, a->h0 + bh * N * P, sizeof(double) * N * P);
    if (a->pB0) memcpy(Bt, a->pB0 + bh * N * R, sizeof(double) * N * R);
    if (a->px0) memcpy(xp, a->px0 + bh * P * R, sizeof(double) * P * R);
    if (a->ang0) for (int i = 0; i < NR; ++i) Th[i] = a->ang0[bh * NR + i];
    const int norm = a->bcnorm;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t bth = (b * T + t) * H + h;
        double *thc = Th + (t + 1) * N2;
        for (int i = 0; i < N2; ++i) thc[i] = Th[t * N2 + i] + (i < NR ? a->theta[bth * NR + i] : 0.0);
        for (int r = 0; r < R; ++r) {
            for (int side = 0; side < 2; ++side) {
                const double *raw = (side == 0 ? a->Bm : a->Cm) + bth * N * R + r;
                const double *gain = side == 0 ? a->b_norm_w : a->c_norm_w;
                const double *bias = side == 0 ? a->b_bias : a->c_bias;
                double *hat = (side == 0 ? Bh : Ch) + t * N * R;
                double *rot = (side == 0 ? Bt + (t + 1) * N * R : Ct + t * N * R);
                double rs = 1.0;
                if (norm) {
                    double ms = 0.0;
                    for (int n = 0; n < N; ++n) ms += raw[n * R] * raw[n * R];
                    rs = 1.0 / sqrt(ms / N + a->eps);
                }
                (side == 0 ? rb : rc)[t * R + r] = rs;
                for (int n = 0; n < N; ++n) {
                    double v = norm ? raw[n * R] * rs * (gain ? gain[n] : 1.0) : raw[n * R];
                    if (bias) v += bias[((int64_t)h * R + r) * N + n];
                    hat[n * R + r] = v;
                }
                for (int i = 0; i < N2; ++i) {
                    const double c = cos(thc[i]), s = sin(thc[i]);
                    const double u = hat[2 * i * R + r], w = hat[(2 * i + 1) * R + r];
                    rot[2 * i * R + r] = u * c - w * s;
                    rot[(2 * i + 1) * R + r] = u * s + w * c;
                }
            }
        }
        double dt = a->dt[bth], lam = a->lam[bth];
        if (a->dt_softplus) dt = sp(dt + (a->dt_bias ? a->dt_bias[h] : 0.0));
        if (a->lam_sigmoid) lam = sg(lam);
        const double A = a->a_per_token ? a->A[bth] : a->A[h];
        dtv[t] = dt; lmv[t] = lam; Av[t] = A;
        al[t] = exp(dt * A);
        be[t] = al[t] * dt * (1.0 - lam);
        ga[t] = lam * dt;
        const double *xt = a->x + bth * P * R, *xprev = t > 0 ? a->x + (bth - H) * P * R : xp;
        const double *Bc = Bt + (t + 1) * N * R, *Bprev = Bt + t * N * R;
        double *hn = hs + (t + 1) * N * P, *ho = hs + t * N * P;
        for (int n = 0; n < N; ++n)
            for (int p = 0; p < P; ++p) {
                double pv = 0.0, cv = 0.0;
                for (int r = 0; r < R; ++r) {
                    pv += Bprev[n * R + r] * xprev[p * R + r];
                    cv += Bc[n * R + r] * xt[p * R + r];
                }
                hn[n * P + p] = al[t] * ho[n * P + p] + be[t] * pv + ga[t] * cv;
            }
        for (int p = 0; p < P; ++p)
            for (int r = 0; r < R; ++r) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n) acc += hn[n * P + p] * Ct[(t * N + n) * R + r];
                yf[(t * P + p) * R + r] = acc + a->D[h] * xt[p * R + r];
            }
    }

    /* ---- reverse sweep */
    double *hb = calloc((size_t)N * P, sizeof(double));      /* gradient of h_t */
    double *Bbn = calloc((size_t)N * R, sizeof(double));     /* gradient of B~_t (accumulated from t and t+1) */
    double *Bbp = calloc((size_t)N * R, sizeof(double));     /* gradient of B~_{t-1} from token t */
    double *xbn = calloc((size_t)P * R, sizeof(double));     /* gradient of x_t from token t+1 */
    double *Cb = calloc((size_t)N * R, sizeof(double));
    double *yb = calloc((size_t)P * R, sizeof(double));
    double *hatb = calloc((size_t)N, sizeof(double));
    double *thb = calloc((size_t)(N2 > 0 ? N2 : 1), sizeof(double)); /* running sum of Theta gradients */
    if (g->dh1) memcpy(hb, g->dh1 + bh * N * P, sizeof(double) * N * P);
    if (g->dpB1) memcpy(Bbn, g->dpB1 + bh * N * R, sizeof(double) * N * R);
    if (g->dpx1) memcpy(xbn, g->dpx1 + bh * P * R, sizeof(double) * P * R);
    if (g->dang1) for (int i = 0; i < NR; ++i) thb[i] = g->dang1[bh * NR + i];
    for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t bth = (b * T + t) * H + h;
        const double *xt = a->x + bth * P * R, *xprev = t > 0 ? a->x + (bth - H) * P * R : xp;
        const double *Bc = Bt + (t + 1) * N * R, *Bprev = Bt + t * N * R, *Cc = Ct + t * N * R;
        const double *hn = hs + (t + 1) * N * P, *ho = hs + t * N * P;
        /* gate and skip */
        for (int e = 0; e < P * R; ++e) {
            double v = g->dy[bth * P * R + e];
            if (a->z) {
                const double zv = a->z[bth * P * R + e], s = sg(zv);
                if (g->dz) g->dz[bth * P * R + e] = v * yf[t * P * R + e] * (s * (1.0 + zv * (1.0 - s)));
                v *= zv * s;
            }
            yb[e] = v;
            pp->dD[h] += v * xt[e];
        }
        double xb_t[1024];
        for (int e = 0; e < P * R; ++e) xb_t[e] = a->D[h] * yb[e] + xbn[e];
        /* output: hb_t += C~ yb^T ; C~b = h_t yb */
        for (int n = 0; n < N; ++n)
            for (int r = 0; r < R; ++r) {
                double acc = 0.0;
                for (int p = 0; p < P; ++p) {
                    hb[n * P + p] += Cc[n * R + r] * yb[p * R + r];
                    acc += hn[n * P + p] * yb[p * R + r];
                }
                Cb[n * R + r] = acc;
            }
        /* update */
        double gab = 0.0, beb = 0.0, alb = 0.0;
        for (int n = 0; n < N; ++n)
            for (int r = 0; r < R; ++r) {
                double sc = 0.0, sp_ = 0.0;
                for (int p = 0; p < P; ++p) {
                    sc += hb[n * P + p] * xt[p * R + r];
                    sp_ += hb[n * P + p] * xprev[p * R + r];
                }
                Bbn[n * R + r] += ga[t] * sc;
                Bbp[n * R + r] = be[t] * sp_;
                gab += Bc[n * R + r] * sc;
                beb += Bprev[n * R + r] * sp_;
            }
        double xbp[1024];
        for (int p = 0; p < P; ++p)
            for (int r = 0; r < R; ++r) {
                double sc = 0.0, sp_ = 0.0;
                for (int n = 0; n < N; ++n) {
                    sc += hb[n * P + p] * Bc[n * R + r];
                    sp_ += hb[n * P + p] * Bprev[n * R + r];
                }
                xb_t[p * R + r] += ga[t] * sc;
                xbp[p * R + r] = be[t] * sp_;
            }
        for (int e = 0; e < N * P; ++e) alb += hb[e] * ho[e];
        if (g->dx) for (int e = 0; e < P * R; ++e) g->dx[bth * P * R + e] = xb_t[e];
        /* scalars */
        const double dt = dtv[t], lam = lmv[t], A = Av[t], alp = al[t];
        double ddt = alb * alp * A + beb * (be[t] * A + alp * (1.0 - lam)) + gab * lam;
        double dlm = -beb * alp * dt + gab * dt;
        const double dAv = alb * alp * dt + beb * be[t] * dt;
        if (g->mutation == 11) ddt = alb * alp * A + gab * lam; /* planted: beta's dt dependence dropped */
        if (a->a_per_token) { if (g->dA) g->dA[bth] = dAv; }
        else pp->dA[h] += dAv;
        if (a->dt_softplus) {
            const double v = a->dt[bth] + (a->dt_bias ? a->dt_bias[h] : 0.0);
            ddt *= sg(v);
            pp->ddtb[h] += ddt;
        }
        if (a->lam_sigmoid) dlm *= lam * (1.0 - lam);
        if (g->ddt) g->ddt[bth] = ddt;
        if (g->dlam) g->dlam[bth] = dlm;
        /* rotation, norm, bias of B~_t (gradient Bbn complete now) and C~_t */
        const double *thc = Th + (t + 1) * N2;
        for (int side = 0; side < 2; ++side) {
            const double *grad = side == 0 ? Bbn : Cb;
            const double *rot = side == 0 ? Bc : Cc;
            const double *hat = (side == 0 ? Bh : Ch) + t * N * R;
            const double *raw = (side == 0 ? a->Bm : a->Cm) + bth * N * R;
            const double *gain = side == 0 ? a->b_norm_w : a->c_norm_w;
            double *dgain = side == 0 ? pp->dbnw : pp->dcnw;
            double *dbias = side == 0 ? pp->dbb : pp->dcb;
            double *draw = side == 0 ? g->dB : g->dC;
            for (int r = 0; r < R; ++r) {
                for (int i = 0; i < N2; ++i) {
                    const double c = cos(thc[i]), s = sin(thc[i]);
                    const double gu = grad[2 * i * R + r], gv = grad[(2 * i + 1) * R + r];
                    hatb[2 * i] = gu * c + gv * s;
                    hatb[2 * i + 1] = -gu * s + gv * c;
                    if (i < NR) {
                        double cr = rot[2 * i * R + r] * gv - rot[(2 * i + 1) * R + r] * gu;
                        if (g->mutation == 12) cr = -cr; /* planted: angle gradient sign */
                        thb[i] += cr;
                    }
                }
                for (int n = 0; n < N; ++n) dbias[((int64_t)h * R + r) * N + n] += hatb[n];
                const double rs = (side == 0 ? rb : rc)[t * R + r];
                if (norm) {
                    double rbar = 0.0;
                    for (int n = 0; n < N; ++n) {
                        const double gn = gain ? gain[n] : 1.0;
                        dgain[n] += hatb[n] * raw[n * R + r] * rs;
                        rbar += hatb[n] * gn * raw[n * R + r];
                    }
                    for (int n = 0; n < N; ++n) {
                        const double gn = gain ? gain[n] : 1.0;
                        double v = hatb[n] * gn * rs - rbar * rs * rs * rs * raw[n * R + r] / N;
                        if (g->mutation == 13) v = hatb[n] * gn * rs; /* planted: norm factor treated as constant */
                        if (draw) draw[bth * N * R + n * R + r] = v;
                    }
                } else if (draw) {
                    for (int n = 0; n < N; ++n) draw[bth * N * R + n * R + r] = hatb[n];
                }
                (void)hat;
            }
        }
        /* theta_t gradient: every later angle includes theta_t */
        if (g->dtheta) for (int i = 0; i < NR; ++i) g->dtheta[bth * NR + i] = thb[i];
        /* carry to token t-1 */
        for (int e = 0; e < N * P; ++e) hb[e] *= alp;
        memcpy(Bbn, Bbp, sizeof(double) * N * R);
        memcpy(xbn, xbp, sizeof(double) * P * R);
    }
    /* initial state: h_{-1}, B~_{-1}, x_{-1}, Theta_{-1} */
    if (g->dh0) memcpy(g->dh0 + bh * N * P, hb, sizeof(double) * N * P);
    if (g->dpB0) memcpy(g->dpB0 + bh * N * R, Bbn, sizeof(double) * N * R);
    if (g->dpx0) memcpy(g->dpx0 + bh * P * R, xbn, sizeof(double) * P * R);
    if (g->dang0) for (int i = 0; i < NR; ++i) g->dang0[bh * NR + i] = thb[i];
    free(hs); free(Bt); free(Ct); free(Bh); free(Ch); free(rb); free(rc); free(Th); free(al); free(be);
    free(ga); free(dtv); free(lmv); free(Av); free(yf); free(xp); free(hb); free(Bbn); free(Bbp); free(xbn);
    free(Cb); free(yb); free(hatb); free(thb);
}

typedef struct { const m3o_bwd_args *g; int64_t begin, end; partial_t part; } bwork_t;

static void *bworker(void *p) {
    bwork_t *w = (bwork_t *)p;
    for (int64_t s = w->begin; s < w->end; ++s)
        bwd_sequence(w->g, s / w->g->f->nheads, (int)(s % w->g->f->nheads), &w->part);
    return NULL;
}

/* Returns 0 on success, -1 on unsupported sizes. */
int m3o_scan_bwd(const m3o_bwd_args *g) {
    const m3o_args *a = g->f;
    if (a->dstate <= 0 || (a->dstate & 1) || a->dstate > 256 || a->rank < 1 || a->headdim <= 0 ||
        a->nheads <= 0 || a->batch < 0 || a->seqlen < 0 || a->rope_pairs < 0 || a->rope_pairs > a->dstate / 2 ||
        (int64_t)a->headdim * a->rank > 1024)
        return -1;
    const int H = a->nheads, N = a->dstate, R = a->rank;
    const int64_t nseq = a->batch * H;
    int nt = a->nthreads > 0 ? a->nthreads : 1;
    if (nt > nseq) nt = (int)(nseq > 0 ? nseq : 1);
    if (nt > 256) nt = 256;
    pthread_t th[256];
    bwork_t w[256];
    for (int i = 0; i < nt; ++i) {
        w[i].g = g;
        w[i].begin = nseq * i / nt;
        w[i].end = nseq * (i + 1) / nt;
        w[i].part.dA = calloc((size_t)H, sizeof(double));
        w[i].part.dD = calloc((size_t)H, sizeof(double));
        w[i].part.dbnw = calloc((size_t)N, sizeof(double));
        w[i].part.dcnw = calloc((size_t)N, sizeof(double));
        w[i].part.dbb = calloc((size_t)H * R * N, sizeof(double));
        w[i].part.dcb = calloc((size_t)H * R * N, sizeof(double));
        w[i].part.ddtb = calloc((size_t)H, sizeof(double));
    }
    for (int i = 1; i < nt; ++i) pthread_create(&th[i], NULL, bworker, &w[i]);
    bworker(&w[0]);
    for (int i = 1; i < nt; ++i) pthread_join(th[i], NULL);
    /* parameter gradients: sums of the per-thread partials, in thread order */
#define SUMTO(dst, field, cnt)                                             \
    if (dst) {                                                             \
        for (int64_t k = 0; k < (cnt); ++k) (dst)[k] = 0.0;                \
        for (int i = 0; i < nt; ++i)                                       \
            for (int64_t k = 0; k < (cnt); ++k) (dst)[k] += w[i].part.field[k]; \
    }
    if (!a->a_per_token) SUMTO(g->dA, dA, H)
    SUMTO(g->dD, dD, H)
    SUMTO(g->dbnw, dbnw, N)
    SUMTO(g->dcnw, dcnw, N)
    SUMTO(g->dbb, dbb, (int64_t)H * R * N)
    SUMTO(g->dcb, dcb, (int64_t)H * R * N)
    SUMTO(g->ddtb, ddtb, H)
#undef SUMTO
    for (int i = 0; i < nt; ++i) {
        free(w[i].part.dA); free(w[i].part.dD); free(w[i].part.dbnw); free(w[i].part.dcnw);
        free(w[i].part.dbb); free(w[i].part.dcb); free(w[i].part.ddtb);
    }
    return 0;
}
