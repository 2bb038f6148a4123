/*
 * libmamba3 -- the Mamba-3 sequence-mixer scan on AMD MI355X (gfx950).
 *
 * The operation (sources are the pages' titles and sections):
 *
 *   Per batch b and head h, over tokens t = 0 .. T-1:
 *     Theta_t = Theta_{t-1} + theta_t                    cumulative data-dependent angle, per pair
 *     B^_t    = g_B * B_t / sqrt(mean_n B_t^2 + eps) + bias_B      (C^_t likewise)
 *     B~_t    = Rot(Theta_t) B^_t,  C~_t = Rot(Theta_t) C^_t          pair i = components (2i, 2i+1)
 *     alpha_t = exp(dt_t A),  beta_t = alpha_t dt_t (1 - lambda_t),  gamma_t = lambda_t dt_t
 *     h_t     = alpha_t h_{t-1} + beta_t B~_{t-1} x_{t-1}^T + gamma_t B~_t x_t^T
 *     y_t     = C~_t^T h_t + D x_t
 *
 *   - The three-term exponential-trapezoidal recurrence: torchmamba README,
 *     "Models" table (Mamba-3 SISO row) and "Math notes" (M3 SISO).
 *   - alpha from exponential-Euler: same page, "Math notes" (M1).  beta and
 *     gamma are not printed on the pages; the form above is the one under
 *     which the dotLLM streaming fix (PR #136, comment "Mamba-3 streaming
 *     decode") folds the trapezoid into one scan with per-token scale
 *     gamma_t + dt_{t+1}(1 - lambda_{t+1}).
 *   - BC norm, then bias, then rotation; lambda per (token, head); theta per
 *     (token, head, pair): dotLLM PR #136, "Summary" and "Key findings /
 *     design decisions".
 *   - Complex state as accumulated data-dependent rotations of B and C:
 *     torchmamba "Math notes" (M3 SISO, RoPE trick).
 *   - MIMO: B, C and x carry a rank axis R; the (N, P) state is shared and
 *     has no rank axis; every output rank r reads C~_t[:, r]:  torchmamba
 *     "Models" (MIMO row) and "API reference" (cache note).
 *   - The carried decode state (h, previous rotated B, previous x, angle):
 *     torchmamba "API reference" (Mamba3SisoCache(angle, ssm, x_prev,
 *     b_prev)); dotLLM PR #136 "Mamba3State" and k_state / v_state.
 *
 * Options of the canonical Mamba-3 block (m3_shape.flags; all off by default):
 *   M3_FLAG_PARTIAL_ROPE  only pairs 0 .. rope_pairs-1 rotate, the others pass through;
 *                         theta and the carried angle hold rope_pairs values (NR below).
 *                         dotLLM PR #136, real-weight validation comment (rope_fraction 0.5:
 *                         32 rotated pairs of d_state 128) and "Mamba3State" (cum_angle
 *                         [n_head, num_rope_angles]).
 *   M3_FLAG_A_PER_TOKEN   A is a per-(batch, token, head) decay rate [B, T, H]:
 *                         alpha_t = exp(dt_t A_t).  dotLLM PR #136, Stage D3 (per-(T,H) ADT).
 *   M3_FLAG_DT_SOFTPLUS   dt holds raw values; the scan uses softplus(dt + dt_bias[h]).
 *   M3_FLAG_LAM_SIGMOID   lam holds raw values; the scan uses sigmoid(lam).
 *                         Both: dotLLM PR #136, "Stage C" (in_proj split -> softplus/sigmoid).
 *   z != NULL             gated output y = (C~^T h + D x) * silu(z), silu(v) = v sigmoid(v).
 *                         dotLLM PR #136, "Stage C" (D skip -> silu(z) gate).
 *   M3_FLAG_HALF_SPLIT    rotation pair i is components (i, i + N/2) of B, C (and of the
 *                         state's rows) instead of (2i, 2i + 1): the rotate-half layout of
 *                         the canonical block.  torchmamba "Math notes" (RoPE trick on pairs
 *                         of state components); the pages leave the pairing layout open and
 *                         the two differ only by a permutation of N.  The decode step,
 *                         the rank-1 scans at N = 64 or 128 whose state is not split finer
 *                         than their output segments, and the gradient call at N = 64 or
 *                         128 pair natively; other calls permute B, C, gains, biases and
 *                         the state rows into the workspace (one extra pass over B and C).
 *                         The workspace size reported for the flag holds those copies
 *                         whichever route a call takes.
 *
 * Layouts: row-major, contiguous, last index fastest.
 *   x, y, z [B, T, H, P]        MIMO: [B, T, H, P, R]       io dtype
 *   Bm, Cm  [B, T, H, N]        MIMO: [B, T, H, N, R]       io dtype, raw (before the norm)
 *   dt, lam [B, T, H]           float32 (activated: dt > 0, lam in [0, 1]; raw with the flags)
 *   theta   [B, T, H, NR]       float32 per-step angle of pair i (NR = N/2, or rope_pairs)
 *   A       [H]                 float32 (A < 0); [B, T, H] with M3_FLAG_A_PER_TOKEN
 *   D, dt_bias [H]              float32 (dt_bias may be NULL: 0)
 *   b_norm_w, c_norm_w [N]      float32 or NULL (gain 1)
 *   b_bias, c_bias     [H, R, N] float32 or NULL (bias 0)
 *   state: h [B, H, N, P], prev_B [B, H, N, R], prev_x [B, H, P, R], angle [B, H, NR], float32
 *
 * Memory: every pointer is a DEVICE pointer owned by the caller.  The
 * library allocates nothing; the scans take a caller-provided workspace of
 * m3_scan_workspace_bytes() bytes.  All calls are asynchronous on the given
 * HIP stream (a hipStream_t passed as void*; NULL = the null stream) and do
 * not synchronise.  The library keeps no global mutable state, so calls on
 * different streams with different workspaces may run concurrently.
 *
 * Errors: arguments are checked on the host before any launch.  NULL
 * required pointers, bad sizes, odd N, R < 1, unknown flags, rope_pairs
 * outside 0 .. N/2 or pointers that are not 16-byte aligned give M3_EINVAL;
 * sizes outside the supported range give
 * M3_EUNSUPPORTED; a short workspace gives M3_EWORKSPACE; a failed launch
 * gives M3_EHIP.  Values are not checked on the device (NaN propagates).
 */
#ifndef LIBMAMBA3_H
#define LIBMAMBA3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    M3_OK = 0,
    M3_EINVAL = 1,
    M3_EUNSUPPORTED = 2,
    M3_EWORKSPACE = 3,
    M3_EHIP = 4
} m3_status;

typedef enum { M3_F32 = 0, M3_BF16 = 1 } m3_dtype; /* dtype of x, B, C and y */

enum {
    M3_FLAG_BCNORM = 1u << 0,       /* apply the RMSNorm over N to B and C */
    M3_FLAG_PARTIAL_ROPE = 1u << 1, /* rotate only the leading rope_pairs pairs */
    M3_FLAG_A_PER_TOKEN = 1u << 2,  /* A is [B, T, H] */
    M3_FLAG_DT_SOFTPLUS = 1u << 3,  /* dt is raw: use softplus(dt + dt_bias[h]) */
    M3_FLAG_LAM_SIGMOID = 1u << 4,  /* lam is raw: use sigmoid(lam) */
    M3_FLAG_HALF_SPLIT = 1u << 5    /* rotation pairs (i, i + N/2) */
};

typedef struct {
    int64_t batch;   /* B >= 0 */
    int64_t seqlen;  /* T >= 0 (m3_step: must be 1) */
    int32_t nheads;  /* H >= 1 */
    int32_t headdim; /* P, 1 .. 128 */
    int32_t dstate;  /* N, even, 2 .. 128 */
    int32_t rank;    /* R, 1 .. 8 (1 for m3_scan_siso) */
    int32_t chunk;   /* requested tokens per chunk, one of 16, 32, 64, 128 with chunk*R <= 128 (the
                        result does not depend on it).  It is an upper bound: the scan kernels work
                        on blocks of at most 64 (token, rank) rows, so a chunk is processed as
                        min(chunk, 64 / R) tokens (chunk 128 runs as 64-token blocks, and rank R
                        as blocks of 64 / R tokens); the gradient call always uses 64 / R */
    int32_t io;      /* m3_dtype */
    uint32_t flags;  /* M3_FLAG_* */
    float norm_eps;  /* RMSNorm epsilon (1e-5 is the usual value) */
    int32_t rope_pairs; /* with M3_FLAG_PARTIAL_ROPE: rotated pairs, 0 .. N/2 (ignored otherwise) */
} m3_shape;

typedef struct {
    const void *x;                    /* [B, T, H, P(, R)]  io dtype */
    const void *Bm, *Cm;              /* [B, T, H, N(, R)]  io dtype */
    const float *dt, *lam;            /* [B, T, H] */
    const float *theta;               /* [B, T, H, NR]; may be NULL when NR == 0 */
    const float *A;                   /* [H], or [B, T, H] with M3_FLAG_A_PER_TOKEN */
    const float *D;                   /* [H] */
    const float *b_norm_w, *c_norm_w; /* [N] or NULL */
    const float *b_bias, *c_bias;     /* [H, R, N] or NULL */
    const float *dt_bias;             /* [H] or NULL; read only with M3_FLAG_DT_SOFTPLUS */
    const void *z;                    /* gate input laid out like y (io dtype), or NULL: no gate */
    /*
     * MIMO projections by learned per-rank vectors, each [H, R, P] float32, or NULL (absent).
     * torchmamba README, "Math notes", MIMO paragraph (per-head x / y / z expanded by a learned
     * vector: D P + P R parameters rather than D P R); dotLLM PR #136, "What's deferred"
     * (MIMO-in-Block: mimo_x / mimo_z projections and the post-scan rank contraction).
     * m3_scan_mimo, m3_scan_noalloc and m3_step only (M3_EINVAL for m3_scan_siso); the
     * gradient call rejects them (M3_EUNSUPPORTED).
     *   mimo_x: x is rank-free [B, T, H, P]; the scan reads x_r[p] = x[p] mimo_x[h, r, p]
     *           (on the bf16 path x_r is formed in fp32 and rounded once to bf16, as an
     *           unexpanded x arrives; the carried prev_x holds x_r in fp32).
     *   mimo_z: z is rank-free [B, T, H, P]; the gate reads z_r[p] = z[p] mimo_z[h, r, p]
     *           (requires z).
     *   mimo_o: y is [B, T, H, P] = sum_r mimo_o[h, r, p] y_r[p] of the gated per-rank
     *           outputs, rounded once.
     */
    const float *mimo_x, *mimo_z, *mimo_o;
    /*
     * Row strides, in elements, between consecutive tokens (rows b*T + t) of inputs that are
     * slices of a wider buffer, such as the in_proj output [B, T, d_in_proj] of the block
     * (dotLLM PR #136, "Stage C": in_proj GEMM -> split -> ...); 0 = contiguous.  Within a row
     * each tensor keeps its layout above ([H, P(, R)], [H, N(, R)], [H], [H, NR]); a stride
     * must be 0 or at least the row's length and below 2^24.  A_stride applies to a per-token
     * A.  Rows whose byte stride is not a multiple of 16 are read element by element.  The
     * gradient call and the half-split pairing of B and C need contiguous inputs
     * (M3_EUNSUPPORTED otherwise).  y is always contiguous.
     */
    int64_t x_stride, B_stride, C_stride, dt_stride, lam_stride, theta_stride, A_stride, z_stride;
} m3_inputs;

typedef struct {
    float *h;      /* [B, H, N, P] state after the last token, in the rotated frame of Theta */
    float *prev_B; /* [B, H, N, R] B~ of the last token (normalised, biased, rotated; not scaled) */
    float *prev_x; /* [B, H, P, R] x of the last token */
    float *angle;  /* [B, H, NR] cumulative angle Theta of the last token, kept in [0, 2 pi) */
} m3_state;

/* Bytes of workspace m3_scan_siso / m3_scan_mimo need for this shape (0 when T == 0 or B == 0,
 * also with M3_FLAG_HALF_SPLIT: such a call only copies the state).  0 for an invalid shape. */
size_t m3_scan_workspace_bytes(const m3_shape *shape);

/*
 * Chunked scan over T tokens (SISO: rank must be 1).
 *   y:     [B, T, H, P] output, io dtype (bf16 rounded to nearest even).
 *   init:  carried state to start from, or NULL for zeros (all four arrays must be set).
 *   final: where to write the state after the last token, or NULL.  May be the
 *          same arrays as init (in-place streaming).  With T == 0, final = init.
 *   ws:    device workspace of at least m3_scan_workspace_bytes(shape) bytes,
 *          owned by the caller; its contents on entry do not matter.  Calls that
 *          share a workspace must be ordered on one stream.
 * Chunk-parallel SSD form: an intra-chunk quadratic part on the matrix
 * cores and a sequential pass over chunk states (torchmamba "Math notes", M2:
 * chunkwise SSD with a factored inter-chunk carry).
 */
m3_status m3_scan_siso(const m3_shape *shape, const m3_inputs *in, void *y, const m3_state *init,
                       m3_state *final, void *ws, size_t ws_bytes, void *stream);

/*
 * Rank-R MIMO scan: same contract as m3_scan_siso with rank R >= 1 and the
 * rank-axis layouts; x, y [B, T, H, P, R], Bm, Cm [B, T, H, N, R].  Every
 * (token, rank) pair is a row of the chunk (chunk * R rows, at most 128).
 * torchmamba "Models" (MIMO row) and "Math notes" (MIMO: rank-R update on a
 * shared state; a chunk of C_SISO / R tokens).
 */
m3_status m3_scan_mimo(const m3_shape *shape, const m3_inputs *in, void *y, const m3_state *init,
                       m3_state *final, void *ws, size_t ws_bytes, void *stream);

/*
 * One decode step (seqlen must be 1) for any rank R: reads and updates
 * `state` in place (all four arrays required) and writes y [B, 1, H, P(, R)].
 * torchmamba "Quickstart"/"API reference" (step(u_t, cache)); dotLLM PR #136
 * "Mamba-3 streaming decode" (the carried previous B~ and x).
 */
m3_status m3_step(const m3_shape *shape, const m3_inputs *in, void *y, m3_state *state,
                  void *stream);

/* Gradients of a scan (every pointer a device pointer owned by the caller; NULL = not
 * wanted).  Per-element gradients have the shape and layout of their inputs: dx, dB, dC,
 * dz in the io dtype, the rest float32.  ddt and dlam are gradients of dt and lam as
 * passed (of the raw values when M3_FLAG_DT_SOFTPLUS / M3_FLAG_LAM_SIGMOID are set).  dA
 * is [H], or [B, T, H] with M3_FLAG_A_PER_TOKEN.  Parameter gradients (dA per head, dD,
 * d_dt_bias, the gains [N] and biases [H, R, N]) are sums over batch and tokens (and over
 * heads for the gains); they are overwritten, not accumulated. */
typedef struct {
    void *dx, *dB, *dC;
    float *ddt, *dlam, *dtheta;
    float *dA, *dD;
    float *db_norm_w, *dc_norm_w;
    float *db_bias, *dc_bias;
    float *ddt_bias;
    void *dz; /* required when the forward call was gated (in->z != NULL) */
} m3_grads;

/* Bytes of workspace m3_scan_bwd needs for this shape (0 when T == 0). */
size_t m3_scan_bwd_workspace_bytes(const m3_shape *shape);

/*
 * Reverse-mode gradients of m3_scan_siso / m3_scan_mimo (any rank R; the same shape,
 * inputs and options as the forward call).
 *   dy:     [B, T, H, P(, R)] gradient of y, io dtype.
 *   init:   the forward call's initial state, or NULL (zeros).
 *   dfinal: gradients of the forward call's final state, or NULL (zeros).
 *   dinit:  where to write the gradients of the initial state, or NULL.
 * The pages ask for a differentiable scan (torchmamba "Verification": fp64 gradchecks;
 * dotLLM PR #136: a trainable block) but print no backward; this is the adjoint of the
 * chunked forward, recomputing the forward states (no forward activations are stored):
 * chunks of 64 (token, rank) rows; the workspace holds the state before and the adjoint
 * after every chunk (2 * B * H * ceil(T / (64 / R)) * N * P floats) plus per-chunk and
 * per-token partial sums.  The chunk length of the shape is not used.  Gradient pointers
 * in grads may be NULL (not computed), except dz of a gated call.  Parameter gradients
 * are sums in a fixed order (results repeat bit for bit between calls).
 * Errors as for the forward call; T == 0 passes the final state's gradients through.
 */
m3_status m3_scan_bwd(const m3_shape *shape, const m3_inputs *in, const void *dy, const m3_state *init,
                      const m3_state *dfinal, m3_grads *grads, m3_state *dinit, void *ws, size_t ws_bytes,
                      void *stream);

/*
 * Allocation-free variant of m3_scan_mimo (any rank R >= 1; R == 1 is the SISO scan), for
 * callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * m3_scan_mimo, but no workspace argument: the workspace is the library's own static
 * device array of M3_STATIC_SCRATCH_BYTES bytes (one per GPU, held from the library's
 * first call on that GPU until the process ends; its address is looked up once per device).
 * The call allocates nothing and frees nothing.
 *   - A shape whose m3_scan_workspace_bytes() exceeds M3_STATIC_SCRATCH_BYTES gives
 *     M3_EWORKSPACE (64 MiB holds e.g. batch 4 x T 2048 x 16 heads at P = N = 64 with any
 *     rank up to 4, and T 16384 x 32 heads at N 128).
 *   - Every call on a GPU shares that GPU's one scratch array: two calls that may overlap in
 *     time on the same GPU (different streams, or different host threads without ordering)
 *     race on it and give wrong results.  Order them on one stream.  The scratch needs no
 *     clearing (its contents on entry do not matter).
 */
#define M3_STATIC_SCRATCH_BYTES (64u << 20)
m3_status m3_scan_noalloc(const m3_shape *shape, const m3_inputs *in, void *y, const m3_state *init,
                          m3_state *final, void *stream);

/*
 * Device-side checks of a debug build (the library compiled with -DM3_DEBUG:
 * libmamba3_debug.so; for developers of the kernels, not for normal use).  In such a build
 * every kernel checks its block, segment and output indices against the call's sizes; a
 * failed check does not fault the device but counts itself and records its source line.
 * This call synchronises the current device, returns the number of failed checks since the
 * last call in *failed and the largest failing source line in *line (either may be NULL),
 * and clears both.  M3_EUNSUPPORTED in a release build (nothing is checked there);
 * M3_EHIP when the device cannot be read.
 */
m3_status m3_debug_checks(uint32_t *failed, uint32_t *line);

/* Static description of a status code. */
const char *m3_status_str(m3_status status);

/* Library version, e.g. "0.2.0". */
const char *m3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMAMBA3_H */
