// m3_bwd.hip -- gradients of the Mamba-3 trapezoidal scan (reverse mode).
//
// The pages ask for the scan to be differentiable (torchmamba "Verification":
// fp64 gradchecks of the scans; dotLLM PR #136: the block trains); they print
// no backward algorithm.  This is the adjoint of the recurrence, computed in
// the complex-state form of the rotation (torchmamba "Math notes", M3 SISO,
// RoPE trick): per pair i the state g_t = Rot(-Theta_t) h_t evolves as
//     g_t = Q_t (alpha_t g_{t-1} + beta_t b_{t-1} x_{t-1}^T) + gamma_t b_t x_t^T,
//     y_t = sum_i c_t^T g_t + D x_t,        Q_t = Rot(-theta_t),
// with b, c the normalised, biased and *unrotated* B and C, so no cumulative
// angle enters the sweeps.  One workgroup walks one (batch, head) sequence:
//
//   forward sweep  recomputes g_t and emits dc_t = g_t dy_t (the gradient of c)
//                  (and, with the gate, the ungated output for dz);
//   reverse sweep  runs the adjoint  G_{t-1} = alpha_t Q_t^T G_t + c_{t-1} dy_{t-1}^T
//                  and emits db_t, dx_t and the per-token scalars.
//
// The gradients of alpha_t and of the per-step angle need <G_t, g_{t-1}>-type
// inner products; instead of the forward states the reverse sweep carries, per
// pair, the 2x2 matrix K_t = sum_p G_t[:, p] g_t[:, p]^T, which obeys
//     K_{t-1} = Q_t^T E_t + c_{t-1} dc_{t-1}^T,
//     E_t     = (K_t - gamma_t u_t b_t^T) Q_t - beta_t v_t b_{t-1}^T,
//     u_t = G_t x_t,  v_t = G_t x_{t-1}   (sums over p),
// and gives  d log alpha_t = sum_i trace(Q_t^T E_t)  and the local angle
// gradient  F01 - F10  of  F = K_t - gamma_t u_t b_t^T.
//
// Lane layout: lane (wave w, row rho, column cc) owns pairs grp*npl .. of the
// state (grp = 4 w + rho) and columns cc*cpl .. ; sums over columns are row
// all-reduces (DPP), sums over pairs go through per-wave partials in LDS that
// are added once per block of 16 (token, rank) rows.
#include <type_traits>

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

namespace {

constexpr int kRows = 16;  // (token, rank) rows per staged block

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over the 16 lanes of a DPP row, returned to every lane of the row
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    return v;
}
// sum over the four rows of a wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rows_sum4(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

struct BwdLds {
    float *sb, *sx, *sc, *sy, *scb, *sbb, *scs, *sth, *sxg, *sxb, *ssc, *ssp, *srn, *spend, *sred, *sthf;
    __device__ BwdLds(float *s, int N, int P) {
        const int RW = kRows + 8;
        sb = s;                  // [RW][N]  b rows; rows 0..R-1 hold the previous token
        sx = sb + RW * N;        // [RW][P]  x rows; rows 0..R-1 hold the previous token
        sc = sx + RW * P;        // [16][N]  c rows
        sy = sc + kRows * N;     // [16][P]  gated dy rows
        scb = sy + kRows * P;    // [16][N]  gradient of c
        sbb = scb + kRows * N;   // [16][N]  gradient of b
        scs = sbb + kRows * N;   // [16][N/2][2] (cos, sin) of the token's angle step
        sth = scs + kRows * N;   // [16][N/2] local angle gradient
        sxg = sth + kRows * (N / 2);  // [4][16][P] per-wave partials (forward: ungated y; reverse: gamma part of dx)
        sxb = sxg + 4 * kRows * P;    // [4][16][P] reverse: beta part of dx of the previous token
        ssc = sxb + 4 * kRows * P;    // [16][8] per token: alpha, beta, gamma, dt, lambda, A, dsoftplus, dsigmoid
        ssp = ssc + kRows * 8;        // [16][4][4] per-wave partial scalars: dlog(alpha), beta grad, gamma grad
        srn = ssp + kRows * 16;       // [16][2] norm factors (b, c) of the rows
        spend = srn + kRows * 2;      // [8][P] dx pending for the previous block's last token (beta part)
        sred = spend + 8 * P;         // [4][2][N] cross-wave sums of the gain gradients
        sthf = sred + 8 * N;          // [N/2] gradient of the final angle
    }
    static __host__ __device__ size_t floats(int N, int P) {
        const int RW = kRows + 8;
        return (size_t)RW * N + (size_t)RW * P + 4 * kRows * N + kRows * N / 2 + 2 * kRows * P +
               8 * kRows * P + kRows * 8 + kRows * 16 + kRows * 2 + 8 * P + 8 * N + N / 2 + 4;
    }
};

}  // namespace

size_t bwd_lds_bytes(int N, int P, int R) {
    (void)R;
    return sizeof(float) * BwdLds::floats(N, P);
}

namespace {

// Normalised (gain, bias) row of raw B or C: one wave, lanes over n.  Returns the
// norm factor; writes the row to dst[N].
template <class Io>
__device__ __forceinline__ float norm_row(const BwdParams &p, const typename Io::T *raw, int R, const float *gain,
                                          const float *bias, float *dst) {
    const int lane = threadIdx.x & 63, N = p.N;
    const bool norm = (p.flags & kFlagNorm) != 0;
    float v[2], ss = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int n = lane + 64 * k;
        v[k] = n < N ? Io::ld(raw + (int64_t)n * R) : 0.f;
        ss += v[k] * v[k];
    }
    ss = rows_sum4(row_sum16(ss));
    const float rs = norm ? rsqrtf(ss / (float)N + p.eps) : 1.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int n = lane + 64 * k;
        if (n < N) {
            float u = norm ? v[k] * rs * (gain ? gain[n] : 1.f) : v[k];
            if (bias) u += bias[n];
            dst[n] = u;
        }
    }
    return rs;
}

// Gradient of a raw B or C row from the gradient of its normalised row (one wave,
// lanes over n); accumulates the gain and bias gradients of this lane's n.
template <class Io>
__device__ __forceinline__ void norm_row_bwd(const BwdParams &p, const typename Io::T *raw, int R, const float *gain,
                                             float rs, const float *grad, typename Io::T *out, float (&again)[2],
                                             float (&abias)[2]) {
    const int lane = threadIdx.x & 63, N = p.N;
    const bool norm = (p.flags & kFlagNorm) != 0;
    float v[2], gv[2], dot = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int n = lane + 64 * k;
        v[k] = n < N ? Io::ld(raw + (int64_t)n * R) : 0.f;
        gv[k] = n < N ? grad[n] : 0.f;
        const float gn = (n < N && gain) ? gain[n] : 1.f;
        dot += gv[k] * gn * v[k];
        abias[k] += gv[k];
        if (norm) again[k] += gv[k] * v[k] * rs;
    }
    dot = rows_sum4(row_sum16(dot));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int n = lane + 64 * k;
        if (n >= N) continue;
        const float gn = gain ? gain[n] : 1.f;
        const float d = norm ? gv[k] * gn * rs - dot * rs * rs * rs * v[k] / (float)N : gv[k];
        if (out) Io::st(out + (int64_t)n * R, d);
    }
}

// dt and lambda after the optional activations, with the derivatives of the activations
__device__ __forceinline__ void act_scalars(const BwdParams &p, int64_t bth, int h, float &dt, float &lam,
                                            float &ddt_draw, float &dlam_draw) {
    dt = p.dt[bth];
    lam = p.lam[bth];
    ddt_draw = 1.f;
    dlam_draw = 1.f;
    if (p.flags & kFlagDtSoftplus) {
        const float v = dt + (p.dtbias ? p.dtbias[h] : 0.f);
        dt = softplus_f(v);
        ddt_draw = sigmoid_f(v);
    }
    if (p.flags & kFlagLamSigmoid) {
        lam = sigmoid_f(lam);
        dlam_draw = lam * (1.f - lam);
    }
}

// Stage tokens t0 .. t0+Tv-1 (and the previous token's b and x rows).
template <class Io>
__device__ void stage_block(const BwdParams &p, const BwdLds &L, int64_t b, int h, int64_t t0, int Tv, bool want_cb) {
    using ET = typename Io::T;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int N = p.N, P = p.P, R = p.R, N2 = N / 2, NR = p.nr;
    const int64_t T = p.T, H = p.H;
    const int64_t bh = b * H + h;
    // b and x rows, previous token included (rows 0 .. R-1)
    for (int row = w; row < (Tv + 1) * R; row += 4) {
        const int64_t t = t0 - 1 + row / R;
        const int r = row % R;
        float *db = L.sb + row * N, *dx = L.sx + row * P;
        if (t >= 0) {
            const int64_t bth = (b * T + t) * H + h;
            const float rs = norm_row<Io>(p, (const ET *)p.Bm + bth * N * R + r, R, p.bnw,
                                          p.bbias ? p.bbias + ((int64_t)h * R + r) * N : nullptr, db);
            if (row >= R && lane == 0) L.srn[(row - R) * 2 + 0] = rs;
            for (int pc = lane; pc < P; pc += 64) dx[pc] = Io::ld((const ET *)p.x + bth * P * R + (int64_t)pc * R + r);
        } else {
            // the carried previous token: b = Rot(-Theta_init) prev_B, x = prev_x
            for (int i = lane; i < N2; i += 64) {
                float u = 0.f, v = 0.f;
                if (p.pB0) {
                    u = p.pB0[(bh * N + 2 * i) * R + r];
                    v = p.pB0[(bh * N + 2 * i + 1) * R + r];
                }
                if (p.ang0 && i < NR) {
                    float s, c;
                    fast_sincos((float)wrap_2pi((double)p.ang0[bh * NR + i]), s, c);
                    const float u2 = c * u + s * v, v2 = -s * u + c * v;
                    u = u2;
                    v = v2;
                }
                db[2 * i] = u;
                db[2 * i + 1] = v;
            }
            for (int pc = lane; pc < P; pc += 64) dx[pc] = p.px0 ? p.px0[(bh * P + pc) * R + r] : 0.f;
        }
    }
    // c rows, gated dy rows, gradient-of-c rows (reverse sweep)
    for (int q = w; q < Tv * R; q += 4) {
        const int64_t t = t0 + q / R;
        const int r = q % R;
        const int64_t bth = (b * T + t) * H + h;
        const float rs = norm_row<Io>(p, (const ET *)p.Cm + bth * N * R + r, R, p.cnw,
                                      p.cbias ? p.cbias + ((int64_t)h * R + r) * N : nullptr, L.sc + q * N);
        if (lane == 0) L.srn[q * 2 + 1] = rs;
        for (int pc = lane; pc < P; pc += 64) {
            const int64_t o = bth * P * R + (int64_t)pc * R + r;
            float g = Io::ld((const ET *)p.dy + o);
            if (p.z) g *= silu_f(Io::ld((const ET *)p.z + o));
            L.sy[q * P + pc] = g;
        }
        if (want_cb)
            for (int n = lane; n < N; n += 64) L.scb[q * N + n] = p.cbar[((bh * T + t) * N + n) * R + r];
    }
    // per-token scalars and angle steps
    if (tid < Tv) {
        const int64_t bth = (b * T + t0 + tid) * H + h;
        float dt, lam, dsp, dsg;
        act_scalars(p, bth, h, dt, lam, dsp, dsg);
        const float A = (p.flags & kFlagAPerToken) ? p.A[bth] : p.A[h];
        const float al = __expf(dt * A);
        float *s = L.ssc + tid * 8;
        s[0] = al;
        s[1] = al * dt * (1.f - lam);
        s[2] = lam * dt;
        s[3] = dt;
        s[4] = lam;
        s[5] = A;
        s[6] = dsp;
        s[7] = dsg;
    }
    for (int e = tid; e < Tv * N2; e += 256) {
        const int k = e / N2, i = e - k * N2;
        float s = 0.f, c = 1.f;
        if (i < NR) {
            const float th = p.theta[((b * T + t0 + k) * H + h) * (int64_t)NR + i];
            s = __sinf(th);
            c = __cosf(th);
        }
        L.scs[e * 2 + 0] = c;
        L.scs[e * 2 + 1] = s;
    }
}

}  // namespace

template <class Io, int NPLM, int CPLM, int RMAX>
__global__ __launch_bounds__(256) void bwd_seq_kernel(BwdParams p) {
    using ET = typename Io::T;
    extern __shared__ __attribute__((aligned(16))) float smem_f[];
    const int N = p.N, P = p.P, R = RMAX == 1 ? 1 : p.R, N2 = N / 2, NR = p.nr;
    const BwdLds L(smem_f, N, P);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rho = lane >> 4, cc = lane & 15, grp = w * 4 + rho;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H;
    const int h = (int)(bh - b * p.H);
    const int64_t T = p.T, H = p.H;
    const int npl = (N2 + 15) / 16, cpl = (P + 15) / 16;
    const int TBt = kRows / R;
    const int nblk = (int)((T + TBt - 1) / TBt);
    const float Dh = p.D[h];

    // per-lane accumulators of parameter gradients
    float aD = 0.f, aA = 0.f, aDtb = 0.f;
    float gB[2] = {0.f, 0.f}, gC[2] = {0.f, 0.f};       // gain gradients, n = lane, lane + 64
    float bB[2][2] = {{0.f, 0.f}, {0.f, 0.f}};           // bias gradients of ranks w, w + 4
    float bC[2][2] = {{0.f, 0.f}, {0.f, 0.f}};

    // ---------------------------------------------------------------- forward sweep
    float G[NPLM][2][CPLM];
    double th_run[NPLM];  // global angle of this lane's pairs (final angle after the sweep)
#pragma unroll
    for (int j = 0; j < NPLM; ++j) {
        const int i = grp * npl + j;
        th_run[j] = (p.ang0 && j < npl && i < NR) ? (double)p.ang0[bh * NR + i] : 0.0;
        float s0 = 0.f, c0 = 1.f;
        if (th_run[j] != 0.0) fast_sincos((float)wrap_2pi(th_run[j]), s0, c0);
#pragma unroll
        for (int q = 0; q < CPLM; ++q) {
            const int pc = cc * cpl + q;
            float u = 0.f, v = 0.f;
            if (j < npl && q < cpl && i < N2 && pc < P && p.h0) {
                u = p.h0[(bh * N + 2 * i) * P + pc];
                v = p.h0[(bh * N + 2 * i + 1) * P + pc];
            }
            G[j][0][q] = c0 * u + s0 * v;  // g = Rot(-Theta_init) h0
            G[j][1][q] = -s0 * u + c0 * v;
        }
    }
    for (int blk = 0; blk < nblk; ++blk) {
        const int64_t t0 = (int64_t)blk * TBt;
        const int Tv = (int)min((int64_t)TBt, T - t0);
        __syncthreads();
        stage_block<Io>(p, L, b, h, t0, Tv, false);
        __syncthreads();
        for (int k = 0; k < Tv; ++k) {
            const float al = L.ssc[k * 8 + 0], be = L.ssc[k * 8 + 1], ga = L.ssc[k * 8 + 2];
#pragma unroll
            for (int j = 0; j < NPLM; ++j) {
                if (j >= npl) break;
                const int i = grp * npl + j;
                const bool iv = i < N2;
                const float c = iv ? L.scs[(k * N2 + i) * 2] : 1.f, s = iv ? L.scs[(k * N2 + i) * 2 + 1] : 0.f;
                if (iv && i < NR) th_run[j] += (double)p.theta[((b * T + t0 + k) * H + h) * (int64_t)NR + i];
#pragma unroll
                for (int q = 0; q < CPLM; ++q) {
                    if (q >= cpl) break;
                    const int pc = cc * cpl + q;
                    const bool ok = iv && pc < P;
                    float m0 = al * G[j][0][q], m1 = al * G[j][1][q];
                    float a0 = 0.f, a1 = 0.f;
#pragma unroll
                    for (int r = 0; r < RMAX; ++r) {
                        if (r >= R) break;
                        if (ok) {
                            const float xp = L.sx[(k * R + r) * P + pc], xc = L.sx[(R + k * R + r) * P + pc];
                            m0 += be * L.sb[(k * R + r) * N + 2 * i] * xp;
                            m1 += be * L.sb[(k * R + r) * N + 2 * i + 1] * xp;
                            a0 += L.sb[(R + k * R + r) * N + 2 * i] * xc;
                            a1 += L.sb[(R + k * R + r) * N + 2 * i + 1] * xc;
                        }
                    }
                    G[j][0][q] = c * m0 + s * m1 + ga * a0;
                    G[j][1][q] = -s * m0 + c * m1 + ga * a1;
                }
            }
            // gradient of c (sum over columns) and, with the gate, the ungated output (sum over pairs)
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
                if (r >= R) break;
                const int q_ = k * R + r;
#pragma unroll
                for (int j = 0; j < NPLM; ++j) {
                    if (j >= npl) break;
                    const int i = grp * npl + j;
                    float c0 = 0.f, c1 = 0.f;
#pragma unroll
                    for (int q = 0; q < CPLM; ++q) {
                        if (q >= cpl) break;
                        const int pc = cc * cpl + q;
                        const float yv = pc < P ? L.sy[q_ * P + pc] : 0.f;
                        c0 += G[j][0][q] * yv;
                        c1 += G[j][1][q] * yv;
                    }
                    c0 = row_sum16(c0);
                    c1 = row_sum16(c1);
                    if (cc == 0 && i < N2) {
                        L.scb[q_ * N + 2 * i] = c0;
                        L.scb[q_ * N + 2 * i + 1] = c1;
                    }
                }
                if (p.z) {
#pragma unroll
                    for (int q = 0; q < CPLM; ++q) {
                        if (q >= cpl) break;
                        const int pc = cc * cpl + q;
                        float acc = 0.f;
#pragma unroll
                        for (int j = 0; j < NPLM; ++j) {
                            if (j >= npl) break;
                            const int i = grp * npl + j;
                            if (i < N2) acc += L.sc[q_ * N + 2 * i] * G[j][0][q] + L.sc[q_ * N + 2 * i + 1] * G[j][1][q];
                        }
                        acc = rows_sum4(acc);
                        if (rho == 0 && pc < P) L.sxg[(w * kRows + q_) * P + pc] = acc;
                    }
                }
            }
        }
        __syncthreads();
        // the gradient of c is complete: keep it for the reverse sweep, and turn it into dC
        for (int e = tid; e < Tv * R * N; e += 256) {
            const int q_ = e / N, n = e - q_ * N;
            const int64_t t = t0 + q_ / R;
            p.cbar[((bh * T + t) * N + n) * R + q_ % R] = L.scb[q_ * N + n];
        }
        for (int r = w, sl = 0; r < R; r += 4, ++sl) {
            for (int k = 0; k < Tv; ++k) {
                const int q_ = k * R + r;
                const int64_t bth = (b * T + t0 + k) * H + h;
                norm_row_bwd<Io>(p, (const ET *)p.Cm + bth * N * R + r, R, p.cnw, L.srn[q_ * 2 + 1], L.scb + q_ * N,
                                 p.dC ? (ET *)p.dC + bth * N * R + r : nullptr, gC, bC[sl]);
            }
        }
        if (p.z && p.dz) {
            for (int e = tid; e < Tv * R * P; e += 256) {
                const int q_ = e / P, pc = e - q_ * P;
                const int64_t t = t0 + q_ / R;
                const int r = q_ % R;
                const int64_t o = ((b * T + t) * H + h) * P * R + (int64_t)pc * R + r;
                const float yf = L.sxg[(0 * kRows + q_) * P + pc] + L.sxg[(1 * kRows + q_) * P + pc] +
                                 L.sxg[(2 * kRows + q_) * P + pc] + L.sxg[(3 * kRows + q_) * P + pc] +
                                 Dh * L.sx[(R + q_) * P + pc];
                const float zv = Io::ld((const ET *)p.z + o), sgz = sigmoid_f(zv);
                Io::st((ET *)p.dz + o, Io::ld((const ET *)p.dy + o) * yf * sgz * (1.f + zv * (1.f - sgz)));
            }
        }
    }

    // ---------------------------------------------------------------- final state
    // b of the last token (complex form) is in the last staged block: rows R + (Tv-1) R + r
    const int TvL = T > 0 ? (int)(T - (int64_t)(nblk - 1) * TBt) : 0;
    float Gb[NPLM][2][CPLM];
    float K[NPLM][2][2];
    float bpend[RMAX][NPLM][2];
    float thf[NPLM];  // gradient of the final angle
#pragma unroll
    for (int j = 0; j < NPLM; ++j) {
        const int i = grp * npl + j;
        const bool iv = j < npl && i < N2;
        float s0 = 0.f, c0 = 1.f;
        if (iv && i < NR && th_run[j] != 0.0) fast_sincos((float)wrap_2pi(th_run[j]), s0, c0);
        float tj = 0.f, k00 = 0.f, k01 = 0.f, k10 = 0.f, k11 = 0.f;
#pragma unroll
        for (int q = 0; q < CPLM; ++q) {
            const int pc = cc * cpl + q;
            float a = 0.f, bq = 0.f;
            if (iv && q < cpl && pc < P && p.dh1) {
                a = p.dh1[(bh * N + 2 * i) * P + pc];
                bq = p.dh1[(bh * N + 2 * i + 1) * P + pc];
            }
            const float g0 = (q < cpl) ? G[j][0][q] : 0.f, g1 = (q < cpl) ? G[j][1][q] : 0.f;
            // h_final = Rot(Theta_final) g ; <dh, J h_final>
            const float hf0 = c0 * g0 - s0 * g1, hf1 = s0 * g0 + c0 * g1;
            tj += -a * hf1 + bq * hf0;
            // gradient of g_final: Rot(-Theta_final) dh
            const float u0 = c0 * a + s0 * bq, u1 = -s0 * a + c0 * bq;
            Gb[j][0][q] = u0;
            Gb[j][1][q] = u1;
            k00 += u0 * g0;
            k01 += u0 * g1;
            k10 += u1 * g0;
            k11 += u1 * g1;
        }
        K[j][0][0] = row_sum16(k00);
        K[j][0][1] = row_sum16(k01);
        K[j][1][0] = row_sum16(k10);
        K[j][1][1] = row_sum16(k11);
        tj = row_sum16(tj);
        // prev_B of the final state = Rot(Theta_final) b_{T-1}
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
            float u = 0.f, v = 0.f;
            if (r < R && iv && p.dpB1) {
                u = p.dpB1[(bh * N + 2 * i) * R + r];
                v = p.dpB1[(bh * N + 2 * i + 1) * R + r];
            }
            float bl0 = 0.f, bl1 = 0.f;
            if (r < R && iv) {
                bl0 = L.sb[(R + (TvL - 1) * R + r) * N + 2 * i];
                bl1 = L.sb[(R + (TvL - 1) * R + r) * N + 2 * i + 1];
            }
            const float pb0 = c0 * bl0 - s0 * bl1, pb1 = s0 * bl0 + c0 * bl1;
            tj += -u * pb1 + v * pb0;
            bpend[r][j][0] = c0 * u + s0 * v;
            bpend[r][j][1] = -s0 * u + c0 * v;
        }
        if (iv && i < NR && p.dang1) tj += p.dang1[bh * NR + i];
        thf[j] = (iv && i < NR) ? tj : 0.f;
        if (cc == 0 && rho >= 0 && iv) L.sthf[i] = thf[j];
    }
    // dx pending of the last token: the final state's prev_x gradient
    __syncthreads();
    for (int e = tid; e < R * P; e += 256) {
        const int r = e / P, pc = e - r * P;
        L.spend[r * P + pc] = p.dpx1 ? p.dpx1[(bh * P + pc) * R + r] : 0.f;
    }

    // ---------------------------------------------------------------- reverse sweep
    for (int blk = nblk - 1; blk >= 0; --blk) {
        const int64_t t0 = (int64_t)blk * TBt;
        const int Tv = (int)min((int64_t)TBt, T - t0);
        __syncthreads();
        stage_block<Io>(p, L, b, h, t0, Tv, true);
        __syncthreads();
        for (int k = Tv - 1; k >= 0; --k) {
            const float al = L.ssc[k * 8 + 0], be = L.ssc[k * 8 + 1], ga = L.ssc[k * 8 + 2];
            float sq = 0.f, sbe = 0.f, sga = 0.f;  // this lane's pairs' shares of the token scalars
#pragma unroll
            for (int j = 0; j < NPLM; ++j) {
                if (j >= npl) break;
                const int i = grp * npl + j;
                const bool iv = i < N2;
                const float c = iv ? L.scs[(k * N2 + i) * 2] : 1.f, s = iv ? L.scs[(k * N2 + i) * 2 + 1] : 0.f;
                // adjoint input and K update
                float Kj00 = K[j][0][0], Kj01 = K[j][0][1], Kj10 = K[j][1][0], Kj11 = K[j][1][1];
#pragma unroll
                for (int r = 0; r < RMAX; ++r) {
                    if (r >= R) break;
                    const int q_ = k * R + r;
                    const float c0 = iv ? L.sc[q_ * N + 2 * i] : 0.f, c1 = iv ? L.sc[q_ * N + 2 * i + 1] : 0.f;
                    const float d0 = iv ? L.scb[q_ * N + 2 * i] : 0.f, d1 = iv ? L.scb[q_ * N + 2 * i + 1] : 0.f;
                    Kj00 += c0 * d0;
                    Kj01 += c0 * d1;
                    Kj10 += c1 * d0;
                    Kj11 += c1 * d1;
#pragma unroll
                    for (int q = 0; q < CPLM; ++q) {
                        if (q >= cpl) break;
                        const int pc = cc * cpl + q;
                        const float yv = pc < P ? L.sy[q_ * P + pc] : 0.f;
                        Gb[j][0][q] += c0 * yv;
                        Gb[j][1][q] += c1 * yv;
                    }
                }
                // F = K - gamma sum_r u_r b_r^T ;  E = F Q - beta sum_r v_r bprev_r^T
                float F00 = Kj00, F01 = Kj01, F10 = Kj10, F11 = Kj11;
                float V00 = 0.f, V01 = 0.f, V10 = 0.f, V11 = 0.f;  // sum_r v_r bprev_r^T
#pragma unroll
                for (int r = 0; r < RMAX; ++r) {
                    if (r >= R) break;
                    float u0 = 0.f, u1 = 0.f, v0 = 0.f, v1 = 0.f;
#pragma unroll
                    for (int q = 0; q < CPLM; ++q) {
                        if (q >= cpl) break;
                        const int pc = cc * cpl + q;
                        const float xc = pc < P ? L.sx[(R + k * R + r) * P + pc] : 0.f;
                        const float xp = pc < P ? L.sx[(k * R + r) * P + pc] : 0.f;
                        u0 += Gb[j][0][q] * xc;
                        u1 += Gb[j][1][q] * xc;
                        v0 += Gb[j][0][q] * xp;
                        v1 += Gb[j][1][q] * xp;
                    }
                    u0 = row_sum16(u0);
                    u1 = row_sum16(u1);
                    v0 = row_sum16(v0);
                    v1 = row_sum16(v1);
                    const float b0 = iv ? L.sb[(R + k * R + r) * N + 2 * i] : 0.f, b1 = iv ? L.sb[(R + k * R + r) * N + 2 * i + 1] : 0.f;
                    const float p0 = iv ? L.sb[(k * R + r) * N + 2 * i] : 0.f, p1 = iv ? L.sb[(k * R + r) * N + 2 * i + 1] : 0.f;
                    F00 -= ga * u0 * b0;
                    F01 -= ga * u0 * b1;
                    F10 -= ga * u1 * b0;
                    F11 -= ga * u1 * b1;
                    V00 += v0 * p0;
                    V01 += v0 * p1;
                    V10 += v1 * p0;
                    V11 += v1 * p1;
                    // gradient of b_t (complete with the part from token t+1) and the part for b_{t-1}
                    const float qv0 = c * v0 - s * v1, qv1 = s * v0 + c * v1;  // Q^T v
                    sga += b0 * u0 + b1 * u1;
                    sbe += p0 * qv0 + p1 * qv1;
                    float nb0 = 0.f, nb1 = 0.f;
#pragma unroll
                    for (int rr = 0; rr < RMAX; ++rr)
                        if (rr == r) { nb0 = bpend[rr][j][0]; nb1 = bpend[rr][j][1]; }
                    if (cc == 0 && iv) {
                        L.sbb[(k * R + r) * N + 2 * i] = nb0 + ga * u0;
                        L.sbb[(k * R + r) * N + 2 * i + 1] = nb1 + ga * u1;
                    }
#pragma unroll
                    for (int rr = 0; rr < RMAX; ++rr)
                        if (rr == r) { bpend[rr][j][0] = be * qv0; bpend[rr][j][1] = be * qv1; }
                }
                if (cc == 0 && iv && i < NR) L.sth[k * N2 + i] = F01 - F10;
                // E = F Q - beta V, with Q = [[c, s], [-s, c]]
                const float E00 = F00 * c - F01 * s - be * V00, E01 = F00 * s + F01 * c - be * V01;
                const float E10 = F10 * c - F11 * s - be * V10, E11 = F10 * s + F11 * c - be * V11;
                // d log alpha share: trace(Q^T E) = sum Q[m][a] E[m][a]
                sq += c * E00 + s * E01 - s * E10 + c * E11;
                // K_{t-1} = Q^T E (the c dc^T term of token t-1 is added at its own step)
                K[j][0][0] = c * E00 - s * E10;
                K[j][0][1] = c * E01 - s * E11;
                K[j][1][0] = s * E00 + c * E10;
                K[j][1][1] = s * E01 + c * E11;
            }
            // dx partials: gamma part for token t, beta part for token t-1 (sums over this lane's pairs)
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
                if (r >= R) break;
                const int q_ = k * R + r;
#pragma unroll
                for (int q = 0; q < CPLM; ++q) {
                    if (q >= cpl) break;
                    const int pc = cc * cpl + q;
                    float xg = 0.f, xb = 0.f;
#pragma unroll
                    for (int j = 0; j < NPLM; ++j) {
                        if (j >= npl) break;
                        const int i = grp * npl + j;
                        if (i >= N2) continue;
                        const float c = L.scs[(k * N2 + i) * 2], s = L.scs[(k * N2 + i) * 2 + 1];
                        const float b0 = L.sb[(R + q_) * N + 2 * i], b1 = L.sb[(R + q_) * N + 2 * i + 1];
                        const float p0 = L.sb[q_ * N + 2 * i], p1 = L.sb[q_ * N + 2 * i + 1];
                        const float qp0 = c * p0 + s * p1, qp1 = -s * p0 + c * p1;  // Q bprev
                        xg += b0 * Gb[j][0][q] + b1 * Gb[j][1][q];
                        xb += qp0 * Gb[j][0][q] + qp1 * Gb[j][1][q];
                    }
                    xg = rows_sum4(xg);
                    xb = rows_sum4(xb);
                    if (rho == 0 && pc < P) {
                        L.sxg[(w * kRows + q_) * P + pc] = ga * xg;
                        L.sxb[(w * kRows + q_) * P + pc] = be * xb;
                    }
                }
            }
            // token scalars: one share per row of lanes
            sq = rows_sum4(cc == 0 ? sq : 0.f);
            sbe = rows_sum4(cc == 0 ? sbe : 0.f);
            sga = rows_sum4(cc == 0 ? sga : 0.f);
            if (lane == 0) {
                L.ssp[(k * 4 + w) * 4 + 0] = sq;
                L.ssp[(k * 4 + w) * 4 + 1] = sbe;
                L.ssp[(k * 4 + w) * 4 + 2] = sga;
            }
            // carry: G <- alpha Q^T G
#pragma unroll
            for (int j = 0; j < NPLM; ++j) {
                if (j >= npl) break;
                const int i = grp * npl + j;
                const bool iv = i < N2;
                const float c = iv ? L.scs[(k * N2 + i) * 2] : 1.f, s = iv ? L.scs[(k * N2 + i) * 2 + 1] : 0.f;
#pragma unroll
                for (int q = 0; q < CPLM; ++q) {
                    if (q >= cpl) break;
                    const float g0 = Gb[j][0][q], g1 = Gb[j][1][q];
                    Gb[j][0][q] = al * (c * g0 - s * g1);
                    Gb[j][1][q] = al * (s * g0 + c * g1);
                }
            }
        }
        __syncthreads();
        // ---- per-token gradients of the block
        if (tid < Tv) {
            const int k = tid;
            const int64_t bth = (b * T + t0 + k) * H + h;
            float qv = 0.f, bb = 0.f, gb = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                qv += L.ssp[(k * 4 + ww) * 4 + 0];
                bb += L.ssp[(k * 4 + ww) * 4 + 1];
                gb += L.ssp[(k * 4 + ww) * 4 + 2];
            }
            const float *sc_ = L.ssc + k * 8;
            const float al = sc_[0], be = sc_[1], dt = sc_[3], lam = sc_[4], A = sc_[5];
            float ddt = qv * A + bb * al * (1.f - lam) * (1.f + dt * A) + gb * lam;
            float dlm = -bb * al * dt + gb * dt;
            const float dAv = qv * dt + bb * be * dt;
            ddt *= sc_[6];
            dlm *= sc_[7];
            if (p.flags & kFlagDtSoftplus) aDtb += ddt;
            if (p.flags & kFlagAPerToken) {
                if (p.dAt) p.dAt[bth] = dAv;
            } else {
                aA += dAv;
            }
            if (p.ddt) p.ddt[bth] = ddt;
            if (p.dlam) p.dlam[bth] = dlm;
        }
        if (p.dtheta)
            for (int e = tid; e < Tv * NR; e += 256) {
                const int k = e / NR, i = e - k * NR;
                p.dtheta[((b * T + t0 + k) * H + h) * (int64_t)NR + i] = L.sth[k * N2 + i] + L.sthf[i];
            }
        // dx: D dy + gamma part + beta part from the next token (or the pending one)
        for (int e = tid; e < Tv * R * P; e += 256) {
            const int q_ = e / P, pc = e - q_ * P;
            const int k = q_ / R, r = q_ - k * R;
            float v = Dh * L.sy[q_ * P + pc];
            aD += L.sy[q_ * P + pc] * L.sx[(R + q_) * P + pc];
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) v += L.sxg[(ww * kRows + q_) * P + pc];
            if (k + 1 < Tv) {
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) v += L.sxb[(ww * kRows + q_ + R) * P + pc];
            } else {
                v += L.spend[r * P + pc];
            }
            if (p.dx) Io::st((ET *)p.dx + ((b * T + t0 + k) * H + h) * P * R + (int64_t)pc * R + r, v);
        }
        // db rows -> dB
        for (int r = w, sl = 0; r < R; r += 4, ++sl) {
            for (int k = 0; k < Tv; ++k) {
                const int q_ = k * R + r;
                const int64_t bth = (b * T + t0 + k) * H + h;
                norm_row_bwd<Io>(p, (const ET *)p.Bm + bth * N * R + r, R, p.bnw, L.srn[q_ * 2 + 0], L.sbb + q_ * N,
                                 p.dB ? (ET *)p.dB + bth * N * R + r : nullptr, gB, bB[sl]);
            }
        }
        __syncthreads();
        // pending dx of the previous block's last token: the beta part produced at this block's first token
        for (int e = tid; e < R * P; e += 256) {
            const int r = e / P, pc = e - r * P;
            float v = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) v += L.sxb[(ww * kRows + r) * P + pc];
            L.spend[r * P + pc] = v;
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- initial state
    // gradient of g_{-1}: Gb;  of b_{-1}: bpend;  of x_{-1}: spend
#pragma unroll
    for (int j = 0; j < NPLM; ++j) {
        const int i = grp * npl + j;
        const bool iv = j < npl && i < N2;
        float s0 = 0.f, c0 = 1.f;
        if (iv && i < NR && p.ang0) fast_sincos((float)wrap_2pi((double)p.ang0[bh * NR + i]), s0, c0);
        float ta = 0.f;
#pragma unroll
        for (int q = 0; q < CPLM; ++q) {
            const int pc = cc * cpl + q;
            if (!(iv && q < cpl && pc < P)) continue;
            const float g0 = Gb[j][0][q], g1 = Gb[j][1][q];
            if (p.dh0) {
                p.dh0[(bh * N + 2 * i) * P + pc] = c0 * g0 - s0 * g1;
                p.dh0[(bh * N + 2 * i + 1) * P + pc] = s0 * g0 + c0 * g1;
            }
            float u = 0.f, v = 0.f;
            if (p.h0) {
                u = p.h0[(bh * N + 2 * i) * P + pc];
                v = p.h0[(bh * N + 2 * i + 1) * P + pc];
            }
            const float gi0 = c0 * u + s0 * v, gi1 = -s0 * u + c0 * v;  // g_{-1}
            ta += g0 * gi1 - g1 * gi0;
        }
        ta = row_sum16(ta);
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
            if (r >= R || !iv) continue;
            const float d0 = bpend[r][j][0], d1 = bpend[r][j][1];
            if (p.dpB0 && cc == 0) {
                p.dpB0[(bh * N + 2 * i) * R + r] = c0 * d0 - s0 * d1;
                p.dpB0[(bh * N + 2 * i + 1) * R + r] = s0 * d0 + c0 * d1;
            }
            const float bi0 = L.sb[r * N + 2 * i], bi1 = L.sb[r * N + 2 * i + 1];  // b_{-1} (staged with block 0)
            ta += d0 * bi1 - d1 * bi0;
        }
        if (p.dang0 && cc == 0 && iv && i < NR) p.dang0[bh * NR + i] = thf[j] + ta;
    }
    if (p.dpx0)
        for (int e = tid; e < R * P; e += 256) {
            const int r = e / P, pc = e - r * P;
            p.dpx0[(bh * P + pc) * R + r] = L.spend[r * P + pc];
        }

    // ---------------------------------------------------------------- parameter partials
    float *part = p.part + bh * (int64_t)p.pw;
    // per-thread scalars -> block sums
    __syncthreads();
    {
        float v0 = rows_sum4(row_sum16(aD)), v1 = rows_sum4(row_sum16(aA)), v2 = rows_sum4(row_sum16(aDtb));
        if (lane == 0) {
            L.sred[w * 4 + 0] = v0;
            L.sred[w * 4 + 1] = v1;
            L.sred[w * 4 + 2] = v2;
        }
    }
    __syncthreads();
    if (tid < 3) part[tid == 0 ? 1 : (tid == 1 ? 0 : 2)] =
        L.sred[0 * 4 + tid] + L.sred[1 * 4 + tid] + L.sred[2 * 4 + tid] + L.sred[3 * 4 + tid];
    __syncthreads();
    // gains: per-wave partials -> sum over waves
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int n = lane + 64 * k;
        if (n < N) {
            L.sred[(w * 2 + 0) * N + n] = gB[k];
            L.sred[(w * 2 + 1) * N + n] = gC[k];
        }
    }
    __syncthreads();
    for (int e = tid; e < 2 * N; e += 256) {
        const int side = e / N, n = e - side * N;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) v += L.sred[(ww * 2 + side) * N + n];
        part[3 + side * N + n] = v;
    }
    // biases: rank r is owned by wave r % 4 (slot r / 4)
    for (int r = w, sl = 0; r < R; r += 4, ++sl) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int n = lane + 64 * k;
            if (n < N) {
                part[3 + 2 * N + r * N + n] = sl == 0 ? bB[0][k] : bB[1][k];
                part[3 + 2 * N + R * N + r * N + n] = sl == 0 ? bC[0][k] : bC[1][k];
            }
        }
    }
    (void)H;
}

// Sums of the per-sequence partials: A (per head), D, dt bias over the batch; gains over
// batch and heads; biases over the batch.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p) {
    const int H = p.H, N = p.N, R = p.R;
    const int64_t Bn = p.B;
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int nH = 3 * H, nG = 2 * N, nBias = 2 * H * R * N;
    if (e < nH) {
        const int which = e / H, h = e - which * H;  // 0: A, 1: D, 2: dt bias
        float *dst = which == 0 ? p.dA : (which == 1 ? p.dD : p.ddtb);
        if (!dst) return;
        float v = 0.f;
        for (int64_t b = 0; b < Bn; ++b) v += p.part[(b * H + h) * (int64_t)p.pw + which];
        dst[h] = v;
    } else if (e < nH + nG) {
        const int k = e - nH, side = k / N, n = k - side * N;
        float *dst = side == 0 ? p.dbnw : p.dcnw;
        if (!dst) return;
        float v = 0.f;
        for (int64_t s = 0; s < Bn * H; ++s) v += p.part[s * p.pw + 3 + side * N + n];
        dst[n] = v;
    } else if (e < nH + nG + nBias) {
        const int k = e - nH - nG, side = k / (H * R * N), rem = k - side * (H * R * N);
        const int h = rem / (R * N), rn = rem - h * (R * N);
        float *dst = side == 0 ? p.dbb : p.dcb;
        if (!dst) return;
        float v = 0.f;
        for (int64_t b = 0; b < Bn; ++b) v += p.part[(b * H + h) * (int64_t)p.pw + 3 + 2 * N + side * R * N + rn];
        dst[(int64_t)h * R * N + rn] = v;
    }
}

// T == 0: the initial state's gradients are the final state's, every parameter gradient is 0.
__global__ __launch_bounds__(256) void bwd_empty_kernel(BwdParams p) {
    const int64_t nbh = p.B * p.H;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int N = p.N, P = p.P, R = p.R, H = p.H;
    if (p.dh0 && e < nbh * N * P) p.dh0[e] = p.dh1 ? p.dh1[e] : 0.f;
    if (p.dpB0 && e < nbh * N * R) p.dpB0[e] = p.dpB1 ? p.dpB1[e] : 0.f;
    if (p.dpx0 && e < nbh * P * R) p.dpx0[e] = p.dpx1 ? p.dpx1[e] : 0.f;
    if (p.dang0 && e < nbh * p.nr) p.dang0[e] = p.dang1 ? p.dang1[e] : 0.f;
    if (e < H) {
        if (p.dA && !(p.flags & kFlagAPerToken)) p.dA[e] = 0.f;
        if (p.dD) p.dD[e] = 0.f;
        if (p.ddtb) p.ddtb[e] = 0.f;
    }
    if (e < N) {
        if (p.dbnw) p.dbnw[e] = 0.f;
        if (p.dcnw) p.dcnw[e] = 0.f;
    }
    if (e < (int64_t)H * R * N) {
        if (p.dbb) p.dbb[e] = 0.f;
        if (p.dcb) p.dcb[e] = 0.f;
    }
}

template <class Io>
static hipError_t launch_bwd_t(const BwdParams &p, hipStream_t st) {
    const size_t lds = bwd_lds_bytes(p.N, p.P, p.R);
    const bool big = (p.N / 2 + 15) / 16 > 2 || (p.P + 15) / 16 > 4;
    const dim3 grid((unsigned)(p.B * p.H)), blk(256);
#define M3_BWD_LAUNCH(NPLM, CPLM, RMAX)                                                                      \
    do {                                                                                                     \
        auto kern = bwd_seq_kernel<Io, NPLM, CPLM, RMAX>;                                                    \
        if (lds > 65536) {                                                                                   \
            hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                               (int)lds);                                                    \
            if (e != hipSuccess) return e;                                                                   \
        }                                                                                                    \
        hipLaunchKernelGGL(kern, grid, blk, lds, st, p);                                                     \
    } while (0)
    if (p.B * p.H > 0 && p.T > 0) {
        if (big) {
            if (p.R == 1) M3_BWD_LAUNCH(4, 8, 1); else M3_BWD_LAUNCH(4, 8, 8);
        } else {
            if (p.R == 1) M3_BWD_LAUNCH(2, 4, 1); else M3_BWD_LAUNCH(2, 4, 8);
        }
    }
#undef M3_BWD_LAUNCH
    return hipGetLastError();
}

hipError_t launch_bwd(bool bf16, const BwdParams &p, hipStream_t st) {
    if (p.T == 0) {
        const int64_t nbh = p.B * p.H;
        int64_t m = nbh * p.N * p.P;
        const int64_t others[] = {nbh * p.N * p.R, nbh * p.P * p.R, (int64_t)p.H * p.R * p.N, p.N, p.H};
        for (int64_t o : others) m = o > m ? o : m;
        if (m > 0) hipLaunchKernelGGL(bwd_empty_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, p);
        return hipGetLastError();
    }
    hipError_t e = bf16 ? launch_bwd_t<IoBF16>(p, st) : launch_bwd_t<IoF32>(p, st);
    if (e != hipSuccess) return e;
    const int total = 3 * p.H + 2 * p.N + 2 * p.H * p.R * p.N;
    if (p.B * p.H > 0 && p.T > 0) {
        hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace m3
