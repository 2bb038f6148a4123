/*
 * m3_oracle.c -- plain fp64 CPU reference of the Mamba-3 trapezoidal selective
 * scan (SISO and rank-R MIMO, complex state as data-dependent RoPE on B/C).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this.  It shares no code with the HIP
 * library and is deliberately slow: one sequential loop over tokens per
 * (batch, head) sequence, everything in double precision.
 *
 * What it computes (sources, by page and section):
 *  - Recurrence  h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1}^T + gamma_t B_t x_t^T,
 *    output y_t = C_t^T h_t (+ D x_t):  torchmamba README, "Models" table
 *    (Mamba-3 SISO row: 3-term trapezoid) and "Math notes" (M3 SISO:
 *    exponential-trapezoidal recurrence with data-dependent lambda).
 *  - alpha = exp(dt*A) (exponential-Euler): torchmamba "Math notes", M1.
 *    beta = alpha*dt*(1-lambda), gamma = lambda*dt: not printed on any page.
 *    Reading taken: the deferred boundary term of the dotLLM streaming fix
 *    ("Mamba-3 streaming decode" comment, PR #136) adds dt_0*(1-lambda_0)*
 *    k_state*v_state to the state *before* the scan decays it, and the
 *    scan's per-token scale is gamma + dt_{t+1}(1-lambda_{t+1}); both hold
 *    only if beta carries the factor alpha.  lambda = 1 then gives the
 *    Mamba-2 update h = alpha h + dt B x^T (torchmamba "Models",
 *    reductions paragraph).
 *  - lambda per token and head; theta per token, head and rotation pair:
 *    dotLLM PR #136, "Key findings / design decisions".
 *  - BC norm (RMSNorm over N), then the per-head bias, then the rotation:
 *    dotLLM PR #136, "Summary" (Mamba3QkNorm, Mamba3DataRoPE) and "Key
 *    findings" (bias after the norm, before RoPE).
 *  - Complex state as accumulated data-dependent pairwise rotations of B
 *    and C: torchmamba "Math notes" (M3 SISO, RoPE trick).  The angle is the
 *    inclusive running sum of theta (the cumulative angle carried in the
 *    decode state, dotLLM "Mamba3State persistent state buffers").  Pair i
 *    is the components (2i, 2i+1); the rotation is the standard
 *    (u, v) -> (u cos a - v sin a, u sin a + v cos a).
 *  - MIMO: rank-R update on a shared (N, P) state; B, C, x carry the rank
 *    axis, theta/dt/lambda/A/D do not (torchmamba "Models" MIMO row,
 *    "API reference" cache note: the state has no R axis).
 *  - Carried state (h, previous rotated B, previous x, cumulative angle):
 *    torchmamba "API reference" (Mamba3SisoCache(angle, ssm, x_prev,
 *    b_prev)); dotLLM "Mamba3State" / k_state, v_state.
 *
 * Options of the canonical block (all off by default):
 *  - Partial rotation: only pairs 0 .. rope_pairs-1 rotate; theta and the
 *    carried angle hold rope_pairs values per (token, head) and the other
 *    pairs pass through unrotated.  dotLLM PR #136, real-weight validation
 *    comment (rope_fraction 0.5 -> num_rope_angles 32 of d_state 128) and
 *    "Mamba3State persistent state buffers" (cum_angle [n_head,
 *    num_rope_angles]).  Which pairs rotate is not printed; reading taken:
 *    the leading ones.
 *  - Per-token decay rate: A indexed per (batch, token, head) instead of per
 *    head, alpha_t = exp(dt_t A_t).  dotLLM PR #136, Stage D3 comment
 *    (per-(T,H) ADT from dd_A).
 *  - Input activations: dt_t = softplus(dt_raw + dt_bias[h]) and
 *    lambda_t = sigmoid(lambda_raw), applied to every token the recurrence
 *    reads (the current, the next one through beta, and token 0 of a
 *    continued call).  dotLLM PR #136, "Stage C" (in_proj split ->
 *    softplus/sigmoid -> Discretize).  The bias inside the softplus is the
 *    usual Mamba dt bias; the pages name the activation only.
 *  - Output gate: y_t = (C_t^T h_t + D x_t) * silu(z_t), silu(v) = v sigmoid(v),
 *    z laid out like y.  dotLLM PR #136, "Stage C" (SelectiveScan -> D skip
 *    -> silu(z) gate).
 *  - MIMO projections by learned per-rank vectors (torchmamba "Math notes",
 *    MIMO paragraph: per-head x / y / z expanded by a learned vector, D P + P R
 *    parameters rather than D P R; dotLLM PR #136, "What's deferred",
 *    MIMO-in-Block: mimo_x / mimo_z projections and the post-scan rank
 *    contraction): with mimo_x the input x is rank-free [.., P] and the scan
 *    reads x_r = x * mimo_x[h, r, :]; with mimo_z the gate reads
 *    z_r = z * mimo_z[h, r, :]; with mimo_o the output is the rank
 *    contraction y = sum_r mimo_o[h, r, :] * y_r of the gated per-rank
 *    outputs.  The carried previous x holds the expanded x_r.
 *
 * Layouts (row-major, last index fastest):
 *   x, y, z [B, T, H, P, R]   B, C [B, T, H, N, R]     dt, lam [B, T, H]
 *   theta [B, T, H, NR]       A [H] (per token: [B, T, H])   D, dt_bias [H]
 *   norm gains [N]            biases [H, R, N]         h [B, H, N, P]
 *   prev_B [B, H, N, R]       prev_x [B, H, P, R]      angle [B, H, NR]
 * with NR = rope_pairs (N/2 unless the rotation is partial).
 * SISO is R = 1 (the trailing unit axis is simply absent in memory).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "m3_oracle.h"

static double softplus(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* dt and lambda of token index `bth` = (b, t, h) after the optional activations */
static double dt_of(const m3o_args *a, int64_t bth, int h) {
    double v = a->dt[bth];
    if (a->dt_softplus) v = softplus(v + (a->dt_bias ? a->dt_bias[h] : 0.0));
    return v;
}
static double lam_of(const m3o_args *a, int64_t bth) {
    double v = a->lam[bth];
    if (a->lam_sigmoid) v = sigmoid(v);
    return v;
}

/* normalise + bias + rotate one raw vector v[N] (stride `stride`) */
static void prep_vec(const m3o_args *a, const double *v, int64_t stride, const double *gain,
                     const double *bias, const double *ang, double *out) {
    const int N = a->dstate;
    double s = 1.0;
    if (a->bcnorm) {
        double ms = 0.0;
        for (int n = 0; n < N; ++n) ms += v[n * stride] * v[n * stride];
        ms /= (double)N;
        s = 1.0 / sqrt(ms + a->eps);
    }
    double hat[256];
    for (int n = 0; n < N; ++n) {
        double g = (a->bcnorm && gain) ? gain[n] : 1.0;
        hat[n] = (a->bcnorm ? g * v[n * stride] * s : v[n * stride]) + (bias ? bias[n] : 0.0);
    }
    for (int i = 0; i < N / 2; ++i) {
        double c = cos(ang[i]), sn = sin(ang[i]);
        if (a->mutation == 3) sn = -sn; /* planted: rotation in the other direction for B and C */
        /* the two components of pair i: adjacent, or one in each half of N */
        const int i0 = a->half_split ? i : 2 * i, i1 = a->half_split ? i + N / 2 : 2 * i + 1;
        double u = hat[i0], w = hat[i1];
        out[i0] = u * c - w * sn;
        out[i1] = u * sn + w * c;
    }
}

static void run_sequence(const m3o_args *a, int64_t b, int h) {
    const int64_t T = a->seqlen;
    const int H = a->nheads, P = a->headdim, N = a->dstate, R = a->rank, N2 = N / 2;
    double *st = calloc((size_t)N * P, sizeof(double));       /* h          [N][P] */
    double *pB = calloc((size_t)N * R, sizeof(double));       /* prev B~    [N][R] */
    double *px = calloc((size_t)P * R, sizeof(double));       /* prev x     [P][R] */
    double *Bt = calloc((size_t)N * R, sizeof(double));       /* B~_t       [N][R] */
    double *Ct = calloc((size_t)N * R, sizeof(double));       /* C~_t       [N][R] */
    const int NR = a->rope_pairs; /* rotated pairs */
    double *ang = calloc((size_t)(N2 > 0 ? N2 : 1), sizeof(double)); /* pairs >= NR stay 0 */
    double *col = calloc((size_t)N, sizeof(double));
    double *xe = calloc((size_t)P * R, sizeof(double));        /* expanded x_t [P][R] */
    const int64_t bh = b * H + h;
    if (a->h0) memcpy(st, a->h0 + bh * N * P, sizeof(double) * N * P);
    if (a->pB0) memcpy(pB, a->pB0 + bh * N * R, sizeof(double) * N * R);
    if (a->px0) memcpy(px, a->px0 + bh * P * R, sizeof(double) * P * R);
    if (a->ang0) memcpy(ang, a->ang0 + bh * NR, sizeof(double) * NR);

    for (int64_t t = 0; t < T; ++t) {
        const int64_t bth = (b * T + t) * H + h; /* index of (b, t, h) */
        /* cumulative angle, inclusive of this token */
        double ang_used[128];
        for (int i = 0; i < N2; ++i) {
            if (i < NR) {
                ang[i] += a->theta[bth * NR + i];
                ang_used[i] = ang[i];
                if (a->mutation == 2) ang_used[i] -= a->theta[bth * NR + i]; /* planted: exclusive sum */
            } else {
                ang_used[i] = 0.0;
            }
        }
        if (a->mutation == 7 && NR > 0 && NR < N2) { /* planted: the trailing pairs rotate instead */
            for (int i = N2 - 1; i >= 0; --i) ang_used[i] = i >= N2 - NR ? ang_used[i - (N2 - NR)] : 0.0;
        }
        for (int r = 0; r < R; ++r) {
            const double *bb = a->b_bias ? a->b_bias + ((int64_t)h * R + r) * N : NULL;
            const double *cb = a->c_bias ? a->c_bias + ((int64_t)h * R + r) * N : NULL;
            prep_vec(a, a->Bm + bth * N * R + r, R, a->b_norm_w, bb, ang_used, col);
            for (int n = 0; n < N; ++n) Bt[n * R + r] = col[n];
            prep_vec(a, a->Cm + bth * N * R + r, R, a->c_norm_w, cb, ang_used, col);
            for (int n = 0; n < N; ++n) Ct[n * R + r] = col[n];
        }
        const double dt = dt_of(a, bth, h), lam = lam_of(a, bth);
        double Av = a->a_per_token ? a->A[bth] : a->A[h];
        if (a->mutation == 6 && a->a_per_token && t > 0) Av = a->A[bth - H]; /* planted: previous token's A */
        const double alpha = exp(dt * Av);
        double beta = alpha * dt * (1.0 - lam);
        double gamma = lam * dt;
        if (a->mutation == 1) beta = dt * (1.0 - lam); /* planted: beta without alpha */
        if (a->mutation == 5) { double tmp = beta; beta = gamma; gamma = tmp; } /* planted: swapped */
        /* x_t per rank: given, or expanded from the rank-free x by the learned vectors */
        const double *xt = a->x + bth * P * R;
        if (a->mimo_x) {
            for (int p = 0; p < P; ++p)
                for (int r = 0; r < R; ++r) xe[p * R + r] = a->x[bth * P + p] * a->mimo_x[((int64_t)h * R + r) * P + p];
            xt = xe;
        }
        /* state update */
        for (int n = 0; n < N; ++n) {
            for (int p = 0; p < P; ++p) {
                double prev_term = 0.0, cur_term = 0.0;
                for (int r = 0; r < R; ++r) {
                    /* planted (mutation 4): pair the previous x with the current B~ */
                    const double *pb = (a->mutation == 4) ? Bt : pB;
                    prev_term += pb[n * R + r] * px[p * R + r];
                    cur_term += Bt[n * R + r] * xt[p * R + r];
                }
                st[n * P + p] = alpha * st[n * P + p] + beta * prev_term + gamma * cur_term;
            }
        }
        /* output: y_t[:, r] = h^T C~_t[:, r] + D x_t[:, r] (gated), or its rank contraction */
        double *yt = a->y + bth * P * (a->mimo_o ? 1 : R);
        for (int p = 0; p < P; ++p) {
            double ysum = 0.0;
            for (int r = 0; r < R; ++r) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n) acc += st[n * P + p] * Ct[n * R + r];
                double v = acc + a->D[h] * xt[p * R + r];
                if (a->z) {
                    const double zv = a->mimo_z ? a->z[bth * P + p] * a->mimo_z[((int64_t)h * R + r) * P + p]
                                                : a->z[bth * P * R + p * R + r];
                    v *= a->mutation == 8 ? sigmoid(zv) : zv * sigmoid(zv); /* planted (8): sigmoid gate */
                }
                if (a->mimo_o) ysum += a->mimo_o[((int64_t)h * R + r) * P + p] * v;
                else yt[p * R + r] = v;
            }
            if (a->mimo_o) yt[p] = ysum;
        }
        memcpy(pB, Bt, sizeof(double) * N * R);
        for (int i = 0; i < P * R; ++i) px[i] = xt[i];
    }
    if (a->h1) memcpy(a->h1 + bh * N * P, st, sizeof(double) * N * P);
    if (a->pB1) memcpy(a->pB1 + bh * N * R, pB, sizeof(double) * N * R);
    if (a->px1) memcpy(a->px1 + bh * P * R, px, sizeof(double) * P * R);
    if (a->ang1) memcpy(a->ang1 + bh * NR, ang, sizeof(double) * NR);
    free(st); free(pB); free(px); free(Bt); free(Ct); free(ang); free(col); free(xe);
}

typedef struct { const m3o_args *a; int64_t begin, end; } work_t;

static void *worker(void *p) {
    work_t *w = (work_t *)p;
    for (int64_t s = w->begin; s < w->end; ++s)
        run_sequence(w->a, s / w->a->nheads, (int)(s % w->a->nheads));
    return NULL;
}

/* Returns 0 on success, -1 on unsupported sizes. */
int m3o_scan(const m3o_args *a) {
    if (a->dstate <= 0 || (a->dstate & 1) || a->dstate > 256 || a->rank < 1 || a->headdim <= 0 ||
        a->nheads <= 0 || a->batch < 0 || a->seqlen < 0 || a->rope_pairs < 0 || a->rope_pairs > a->dstate / 2)
        return -1;
    const int64_t nseq = a->batch * a->nheads;
    int nt = a->nthreads > 0 ? a->nthreads : 1;
    if (nt > nseq) nt = (int)(nseq > 0 ? nseq : 1);
    pthread_t th[256];
    work_t w[256];
    if (nt > 256) nt = 256;
    for (int i = 0; i < nt; ++i) {
        w[i].a = a;
        w[i].begin = nseq * i / nt;
        w[i].end = nseq * (i + 1) / nt;
    }
    for (int i = 1; i < nt; ++i) pthread_create(&th[i], NULL, worker, &w[i]);
    worker(&w[0]);
    for (int i = 1; i < nt; ++i) pthread_join(th[i], NULL);
    return 0;
}
