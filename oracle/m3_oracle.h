/*
 * m3_oracle.h -- argument block of the fp64 oracle (m3_oracle.c forward,
 * m3_oracle_bwd.c backward).  TEST INFRASTRUCTURE ONLY; not used by the HIP
 * library.
 */
#ifndef M3_ORACLE_H
#define M3_ORACLE_H
#include <stdint.h>

typedef struct {
    int64_t batch, seqlen;
    int32_t nheads, headdim, dstate, rank;
    int32_t bcnorm;       /* 1: RMSNorm over N on B and C before the bias */
    double eps;           /* RMSNorm epsilon */
    /* inputs (NULL where optional) */
    const double *x, *Bm, *Cm, *dt, *lam, *theta, *A, *D;
    const double *b_norm_w, *c_norm_w;   /* [N] or NULL (= 1) */
    const double *b_bias, *c_bias;       /* [H, R, N] or NULL (= 0) */
    const double *h0, *pB0, *px0, *ang0; /* initial state or NULL (= 0) */
    /* outputs */
    double *y;                            /* [B, T, H, P, R] */
    double *h1, *pB1, *px1, *ang1;        /* final state or NULL */
    /* Test hook: a nonzero value plants one deliberate mistake so that the
     * pin tests can show they catch it.  0 in every real use. */
    int32_t mutation;
    int32_t nthreads;
    /* canonical-block options */
    int32_t rope_pairs;   /* rotated pairs (0 .. N/2); theta [B,T,H,rope_pairs], angle [B,H,rope_pairs] */
    int32_t a_per_token;  /* 1: A is [B, T, H] */
    int32_t dt_softplus;  /* 1: dt holds raw values; dt = softplus(dt + dt_bias[h]) */
    int32_t lam_sigmoid;  /* 1: lam holds raw values; lambda = sigmoid(lam) */
    const double *dt_bias; /* [H] or NULL (= 0) */
    const double *z;       /* gate input laid out like y, or NULL (no gate) */
    int32_t half_split;    /* 1: pair i is components (i, i + N/2); 0: (2i, 2i + 1) */
    /* MIMO projections by learned per-rank vectors [H, R, P] (NULL = absent):
     *   mimo_x: x is [B, T, H, P] and the scan reads x_r[p] = x[p] mimo_x[h, r, p];
     *   mimo_z: z is [B, T, H, P] and the gate reads z_r[p] = z[p] mimo_z[h, r, p];
     *   mimo_o: y is [B, T, H, P] = sum_r mimo_o[h, r, p] y_r[p] (y_r after the gate). */
    const double *mimo_x, *mimo_z, *mimo_o;
} m3o_args;

int m3o_scan(const m3o_args *a);

#endif
