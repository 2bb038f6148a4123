// m3_bwd.hip -- gradients of the Mamba-3 trapezoidal scan (reverse mode).
//
// The pages ask for the scan to be differentiable (torchmamba "Verification":
// fp64 gradchecks of the scans; dotLLM PR #136: the block trains); they print
// no backward algorithm.  This is the adjoint of the recurrence, computed in
// the complex-state form of the rotation (torchmamba "Math notes", M3 SISO,
// RoPE trick): per pair i the state g_t = Rot(-Theta_t) h_t evolves as
//     g_t = Q_t (alpha_t g_{t-1} + beta_t b_{t-1} x_{t-1}^T) + gamma_t b_t x_t^T,
//     y_t = sum_i c_t^T g_t + D x_t,        Q_t = Rot(-theta_t),
// with b, c the normalised, biased and unrotated B and C, so no cumulative
// angle enters the sweeps.  The adjoint is
//     G_{t-1} = alpha_t Q_t^T G_t + c_{t-1} dy_{t-1}^T,
// and the decay and angle gradients, which need <G_t, g_{t-1}>-type inner
// products, come from the per-pair 2x2 matrix K_t = sum_p G_t[:, p] g_t[:, p]^T:
//     K_{t-1} = Q_t^T E_t + c_{t-1} dc_{t-1}^T,
//     E_t     = (K_t - gamma_t u_t b_t^T) Q_t - beta_t v_t b_{t-1}^T,
//     u_t = G_t x_t,  v_t = G_t x_{t-1},  dc_t = g_t dy_t   (sums over the columns p),
//     d log alpha_t = sum_i trace(Q_t^T E_t),  local angle gradient = F01 - F10 of
//     F = K_t - gamma_t u_t b_t^T.
//
// Every quantity above is linear in the per-column contributions, and the
// state columns evolve independently, so a workgroup handles one group of 16
// columns of one time segment of one (batch, head) sequence; partial sums over
// the column groups are added by the final per-token kernel.  Segments are
// chained like the forward's: forward aggregates from zero, a fold that turns
// them into segment start states; reverse aggregates of the adjoint from zero,
// a fold that turns them into segment end adjoints.  Kernels, in launch order:
//   bwd_sweep_kernel (mode 0)  forward aggregate of each segment
//   bwd_ffold_kernel           segment start states, final angle
//   bwd_sweep_kernel (mode 1)  adjoint aggregate of each segment
//   bwd_rfold_kernel           segment end adjoints, gradient of the initial h
//   bwd_sweep_kernel (mode 2)  both sweeps of each segment: column-group shares
//   bwd_final_kernel           per-token sums, norm backward, boundary terms
//   bwd_reduce_kernel          parameter gradients
//
// Lane layout of a sweep: lane (wave w, row rho, column cc) owns pairs
// (4 w + rho) * NPL + j of the state and column cc of the group; sums over
// columns are row all-reduces (DPP), sums over pairs go through per-wave
// partials in LDS added once per block of 16 (token, rank) rows.
#include <type_traits>

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

namespace {

constexpr int kRows = 16;  // (token, rank) rows per staged block
constexpr int kCW = 16;    // state columns per workgroup

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
__device__ __forceinline__ float wave_sum(float v) { return rows_sum4(row_sum16(v)); }

// Normalised (gain, bias) row of raw B or C: one wave, lanes over n.  Returns the norm
// factor; writes the row to dst[N] (when dst is not NULL).
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
    ss = wave_sum(ss);
    const float rs = norm ? rsqrtf(ss / (float)N + p.eps) : 1.f;
    if (dst) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int n = lane + 64 * k;
            if (n < N) {
                float u = norm ? v[k] * rs * (gain ? gain[n] : 1.f) : v[k];
                if (bias) u += bias[n];
                dst[n] = u;
            }
        }
    }
    return rs;
}

// dt and lambda after the optional activations, with the activations' derivatives
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

// Complex-form b of the carried previous token: Rot(-Theta_init) prev_B (pair i, rank r)
__device__ __forceinline__ void init_b(const BwdParams &p, int64_t bh, int i, int r, float &u, float &v) {
    const int N = p.N, R = p.R;
    u = v = 0.f;
    if (p.pB0) {
        u = p.pB0[(bh * N + 2 * i) * R + r];
        v = p.pB0[(bh * N + 2 * i + 1) * R + r];
    }
    if (p.ang0 && i < p.nr) {
        float s, c;
        fast_sincos((float)wrap_2pi((double)p.ang0[bh * p.nr + i]), s, c);
        const float u2 = c * u + s * v, v2 = -s * u + c * v;
        u = u2;
        v = v2;
    }
}

// LDS layout of the sweep kernel (floats)
template <int NPAD>
struct SweepLds {
    static constexpr int RW = kRows + 8;                // rows incl. the previous token's (R <= 8)
    static constexpr int SB = 0;                        // [RW][NPAD] b rows (rows 0..R-1: previous token)
    static constexpr int SX = SB + RW * NPAD;           // [RW][16]   x rows (own columns)
    static constexpr int SC = SX + RW * kCW;            // [16][NPAD] c rows
    static constexpr int SY = SC + kRows * NPAD;        // [16][16]   gated dy rows
    static constexpr int SCB = SY + kRows * kCW;        // [16][NPAD] gradient of c (share)
    static constexpr int SCS = SCB + kRows * NPAD;      // [16][NPAD/2][2] (cos, sin) of the angle steps
    static constexpr int SXG = SCS + kRows * NPAD;      // [4][16][16] per-wave partials (ungated y / gamma part of dx)
    static constexpr int SXB = SXG + 4 * kRows * kCW;   // [4][16][16] beta part of dx of the previous token
    static constexpr int SSC = SXB + 4 * kRows * kCW;   // [16][8] alpha, beta, gamma, dt, lambda, A, -, -
    static constexpr int SSP = SSC + kRows * 8;         // [16][4][4] per-wave partial scalars
    static constexpr int SPN = SSP + kRows * 16;        // [8][16] dx pending for the previous block's last token
    static constexpr int SRD = SPN + 8 * kCW;           // [8] reductions
    static constexpr int TOTAL = SRD + 8;
};

// Stage tokens t0 .. t0+Tv-1 of one sequence (b and x rows of the previous token too).
// Every global load of the block is issued before the first use, so the block pays
// the memory latency once.
template <class Io, int NPAD>
__device__ void stage(const BwdParams &p, float *sm, int64_t b, int h, int cg, int64_t t0, int Tv, bool want_c,
                      bool want_cb) {
    using ET = typename Io::T;
    using L = SweepLds<NPAD>;
    constexpr int MB = (kRows + 8) / 4, MC = kRows / 4, MT = kRows * (NPAD / 2) / 256 > 0 ? kRows * (NPAD / 2) / 256 : 1;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int N = p.N, P = p.P, R = p.R, N2 = N / 2, NR = p.nr;
    const int64_t T = p.T, H = p.H;
    const int64_t bh = b * H + h;
    const int p0 = cg * kCW;
    const bool norm = (p.flags & kFlagNorm) != 0;
    const int nbr = (Tv + 1) * R, ncr = Tv * R;
    // ---- loads
    float bv[MB][2], xv[MB], cvv[MC][2], yv[MC], zv[MC], cb[MC][2];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int row = w + 4 * m;
        bv[m][0] = bv[m][1] = xv[m] = 0.f;
        const int64_t t = t0 - 1 + row / R;
        if (row < nbr && t >= 0) {
            const int r = row % R;
            const int64_t bth = (b * T + t) * H + h;
            const ET *raw = (const ET *)p.Bm + bth * N * R + r;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int n = lane + 64 * k;
                if (n < N) bv[m][k] = Io::ld(raw + (int64_t)n * R);
            }
            if (lane < kCW && p0 + lane < P) xv[m] = Io::ld((const ET *)p.x + bth * P * R + (int64_t)(p0 + lane) * R + r);
        }
    }
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int q = w + 4 * m;
        cvv[m][0] = cvv[m][1] = yv[m] = cb[m][0] = cb[m][1] = 0.f;
        zv[m] = 1.f;
        if (want_c && q < ncr) {
            const int64_t t = t0 + q / R;
            const int r = q % R;
            const int64_t bth = (b * T + t) * H + h;
            const ET *raw = (const ET *)p.Cm + bth * N * R + r;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int n = lane + 64 * k;
                if (n < N) cvv[m][k] = Io::ld(raw + (int64_t)n * R);
                if (want_cb && n < N) cb[m][k] = p.cbar[((cg * (p.B * H) + bh) * T + t) * (int64_t)N * R + n * R + r];
            }
            if (lane < kCW && p0 + lane < P) {
                const int64_t o = bth * P * R + (int64_t)(p0 + lane) * R + r;
                yv[m] = Io::ld((const ET *)p.dy + o);
                if (p.z) zv[m] = Io::ld((const ET *)p.z + o);
            }
        }
    }
    float sdt = 0.f, slam = 0.f, sA = 0.f;
    if (tid < Tv) {
        const int64_t bth = (b * T + t0 + tid) * H + h;
        sdt = p.dt[bth];
        slam = p.lam[bth];
        sA = (p.flags & kFlagAPerToken) ? p.A[bth] : p.A[h];
    }
    float th[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int e = tid + 256 * m;
        const int k = e / N2, i = e - k * N2;
        th[m] = 0.f;
        if (k < Tv && i < NR) th[m] = p.theta[((b * T + t0 + k) * H + h) * (int64_t)NR + i];
    }
    // ---- normalised rows and the rest
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int row = w + 4 * m;
        if (row >= nbr) continue;  // uniform per wave
        const int64_t t = t0 - 1 + row / R;
        const int r = row % R;
        float *db = sm + L::SB + row * NPAD;
        if (t >= 0) {
            const float ss = wave_sum(bv[m][0] * bv[m][0] + bv[m][1] * bv[m][1]);
            const float rs = norm ? rsqrtf(ss / (float)N + p.eps) : 1.f;
            const float *bias = p.bbias ? p.bbias + ((int64_t)h * R + r) * N : nullptr;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int n = lane + 64 * k;
                if (n < N) {
                    float u = norm ? bv[m][k] * rs * (p.bnw ? p.bnw[n] : 1.f) : bv[m][k];
                    if (bias) u += bias[n];
                    db[n] = u;
                }
            }
            if (lane < kCW) sm[L::SX + row * kCW + lane] = xv[m];
        } else {
            for (int i = lane; i < N2; i += 64) init_b(p, bh, i, r, db[2 * i], db[2 * i + 1]);
            if (lane < kCW) sm[L::SX + row * kCW + lane] = (p.px0 && p0 + lane < P) ? p.px0[(bh * P + p0 + lane) * R + r] : 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int q = w + 4 * m;
        if (!want_c || q >= ncr) continue;  // uniform per wave
        const int r = q % R;
        const float ss = wave_sum(cvv[m][0] * cvv[m][0] + cvv[m][1] * cvv[m][1]);
        const float rs = norm ? rsqrtf(ss / (float)N + p.eps) : 1.f;
        const float *bias = p.cbias ? p.cbias + ((int64_t)h * R + r) * N : nullptr;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int n = lane + 64 * k;
            if (n < N) {
                float u = norm ? cvv[m][k] * rs * (p.cnw ? p.cnw[n] : 1.f) : cvv[m][k];
                if (bias) u += bias[n];
                sm[L::SC + q * NPAD + n] = u;
                if (want_cb) sm[L::SCB + q * NPAD + n] = cb[m][k];
            }
        }
        if (lane < kCW) sm[L::SY + q * kCW + lane] = p.z ? yv[m] * silu_f(zv[m]) : yv[m];
    }
    if (tid < Tv) {
        float dt = sdt, lam = slam;
        if (p.flags & kFlagDtSoftplus) dt = softplus_f(dt + (p.dtbias ? p.dtbias[h] : 0.f));
        if (p.flags & kFlagLamSigmoid) lam = sigmoid_f(lam);
        const float al = __expf(dt * sA);
        float *s = sm + L::SSC + tid * 8;
        s[0] = al;
        s[1] = al * dt * (1.f - lam);
        s[2] = lam * dt;
        s[3] = dt;
        s[4] = lam;
        s[5] = sA;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int e = tid + 256 * m;
        const int k = e / N2, i = e - k * N2;
        if (k >= Tv) continue;
        sm[L::SCS + (k * (NPAD / 2) + i) * 2 + 0] = i < NR ? __cosf(th[m]) : 1.f;
        sm[L::SCS + (k * (NPAD / 2) + i) * 2 + 1] = i < NR ? __sinf(th[m]) : 0.f;
    }
}

}  // namespace

// mode 0: forward aggregate; 1: adjoint aggregate; 2: both sweeps with the shares
template <class Io, int NPAD, int RMAX>
__global__ __launch_bounds__(256) void bwd_sweep_kernel(BwdParams p, int mode) {
    using ET = typename Io::T;
    using L = SweepLds<NPAD>;
    constexpr int N2P = NPAD / 2;
    constexpr int NPL = N2P >= 16 ? N2P / 16 : 1;
    __shared__ __attribute__((aligned(16))) float sm[L::TOTAL];
    const int N = p.N, P = p.P, R = RMAX == 1 ? 1 : p.R, N2 = N / 2, NR = p.nr;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rho = lane >> 4, cc = lane & 15, grp = w * 4 + rho;
    const int64_t bid = blockIdx.x;
    const int seg = (int)(bid % p.nseg);
    const int64_t q1 = bid / p.nseg;
    const int cg = (int)(q1 % p.ncg);
    const int64_t bh = q1 / p.ncg;
    const int64_t b = bh / p.H;
    const int h = (int)(bh - b * p.H);
    const int64_t T = p.T, H = p.H, BH = p.B * p.H;
    const int TBt = kRows / R;
    const int64_t ts = (int64_t)seg * p.segT, te = min(T, ts + (int64_t)p.segT);
    const int nblk = (int)((te - ts + TBt - 1) / TBt);
    const int pc = cg * kCW + cc;  // this lane's column
    const bool cv = pc < P;
    const int64_t sidx = (bh * p.ncg + cg) * p.nseg + seg;  // (sequence, group, segment)
    const int i0 = grp * NPL;
    auto piv = [&](int j) { return i0 + j < N2; };
    auto CS = [&](int k, int i, int c) { return sm[L::SCS + (k * N2P + i) * 2 + c]; };
    auto SB = [&](int row, int n) { return sm[L::SB + row * NPAD + n]; };
    auto SX = [&](int row) { return sm[L::SX + row * kCW + cc]; };

    float G[NPL][2];
#pragma unroll
    for (int j = 0; j < NPL; ++j) G[j][0] = G[j][1] = 0.f;
    // ---------------------------------------------------------------- forward sweep (modes 0, 2)
    if (mode != 1) {
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int i = i0 + j;
            G[j][0] = G[j][1] = 0.f;
            if (mode == 2 && piv(j)) {
                G[j][0] = p.Gagg[(sidx * N + 2 * i) * kCW + cc];
                G[j][1] = p.Gagg[(sidx * N + 2 * i + 1) * kCW + cc];
            }
        }
        for (int blk = 0; blk < nblk; ++blk) {
            const int64_t t0 = ts + (int64_t)blk * TBt;
            const int Tv = (int)min((int64_t)TBt, te - t0);
            __syncthreads();
            stage<Io, NPAD>(p, sm, b, h, cg, t0, Tv, mode == 2, false);
            __syncthreads();
            if (mode == 0) {
                // segment totals of log alpha and of the angle steps (one group writes them)
                if (cg == 0 && tid == 0)
                    for (int k = 0; k < Tv; ++k) lsum += sm[L::SSC + k * 8 + 3] * sm[L::SSC + k * 8 + 5];
            }
            for (int k = 0; k < Tv; ++k) {
                const float al = sm[L::SSC + k * 8 + 0], be = sm[L::SSC + k * 8 + 1], ga = sm[L::SSC + k * 8 + 2];
#pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const int i = i0 + j;
                    if (!piv(j)) continue;
                    const float c = CS(k, i, 0), s = CS(k, i, 1);
                    float m0 = al * G[j][0], m1 = al * G[j][1], a0 = 0.f, a1 = 0.f;
#pragma unroll
                    for (int r = 0; r < RMAX; ++r) {
                        if (r >= R) break;
                        const float xp = SX(k * R + r), xc = SX(R + k * R + r);
                        m0 += be * SB(k * R + r, 2 * i) * xp;
                        m1 += be * SB(k * R + r, 2 * i + 1) * xp;
                        a0 += SB(R + k * R + r, 2 * i) * xc;
                        a1 += SB(R + k * R + r, 2 * i + 1) * xc;
                    }
                    G[j][0] = c * m0 + s * m1 + ga * a0;
                    G[j][1] = -s * m0 + c * m1 + ga * a1;
                }
                if (mode == 2) {
#pragma unroll
                    for (int r = 0; r < RMAX; ++r) {
                        if (r >= R) break;
                        const int q_ = k * R + r;
                        const float yv = sm[L::SY + q_ * kCW + cc];
                        float yt = 0.f;
#pragma unroll
                        for (int j = 0; j < NPL; ++j) {
                            const int i = i0 + j;
                            const float c0 = row_sum16(G[j][0] * yv), c1 = row_sum16(G[j][1] * yv);
                            if (cc == 0 && piv(j)) {
                                sm[L::SCB + q_ * NPAD + 2 * i] = c0;
                                sm[L::SCB + q_ * NPAD + 2 * i + 1] = c1;
                            }
                            if (piv(j)) yt += sm[L::SC + q_ * NPAD + 2 * i] * G[j][0] + sm[L::SC + q_ * NPAD + 2 * i + 1] * G[j][1];
                        }
                        if (p.z) {
                            yt = rows_sum4(yt);
                            if (rho == 0) sm[L::SXG + (w * kRows + q_) * kCW + cc] = yt;
                        }
                    }
                }
            }
            if (mode == 2) {
                __syncthreads();
                // the gradient of c (this group's share) for the reverse sweep and the final kernel
                for (int e = tid; e < Tv * R * N; e += 256) {
                    const int q_ = e / N, n = e - q_ * N;
                    const int64_t t = t0 + q_ / R;
                    p.cbar[((cg * BH + bh) * T + t) * (int64_t)N * R + n * R + q_ % R] = sm[L::SCB + q_ * NPAD + n];
                }
                if (p.z && p.dz) {
                    for (int e = tid; e < Tv * R * kCW; e += 256) {
                        const int q_ = e / kCW, c2 = e - q_ * kCW;
                        if (cg * kCW + c2 >= P) continue;
                        const int64_t t = t0 + q_ / R;
                        const int64_t o = ((b * T + t) * H + h) * P * R + (int64_t)(cg * kCW + c2) * R + q_ % R;
                        float yf = p.D[h] * sm[L::SX + (R + q_) * kCW + c2];
#pragma unroll
                        for (int ww = 0; ww < 4; ++ww) yf += sm[L::SXG + (ww * kRows + q_) * kCW + c2];
                        const float zv = Io::ld((const ET *)p.z + o), sgz = sigmoid_f(zv);
                        Io::st((ET *)p.dz + o, Io::ld((const ET *)p.dy + o) * yf * sgz * (1.f + zv * (1.f - sgz)));
                    }
                }
            }
            if (mode == 0 && cg == 0) {
                // angle totals of the segment, per pair
                for (int i = tid; i < N2; i += 256) {
                    float a = blk == 0 ? 0.f : p.pseg[(bh * p.nseg + seg) * N2 + i];
                    if (i < NR)
                        for (int k = 0; k < Tv; ++k) a += p.theta[((b * T + t0 + k) * H + h) * (int64_t)NR + i];
                    p.pseg[(bh * p.nseg + seg) * N2 + i] = a;
                }
            }
        }
        if (mode == 0) {
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                const int i = i0 + j;
                if (!piv(j)) continue;
                p.Gagg[(sidx * N + 2 * i) * kCW + cc] = G[j][0];
                p.Gagg[(sidx * N + 2 * i + 1) * kCW + cc] = G[j][1];
            }
            if (cg == 0 && tid == 0) p.lseg[bh * p.nseg + seg] = lsum;
            return;
        }
    }

    // ---------------------------------------------------------------- reverse sweep (modes 1, 2)
    float Gb[NPL][2], K[NPL][2][2], bpend[RMAX][NPL][2];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int i = i0 + j;
        Gb[j][0] = Gb[j][1] = 0.f;
        if (mode == 2 && piv(j)) {
            Gb[j][0] = p.Ragg[(sidx * N + 2 * i) * kCW + cc];
            Gb[j][1] = p.Ragg[(sidx * N + 2 * i + 1) * kCW + cc];
        }
#pragma unroll
        for (int r = 0; r < RMAX; ++r) bpend[r][j][0] = bpend[r][j][1] = 0.f;
        // K at the segment end: sum over the columns of G_end g_end^T
        K[j][0][0] = row_sum16(Gb[j][0] * G[j][0]);
        K[j][0][1] = row_sum16(Gb[j][0] * G[j][1]);
        K[j][1][0] = row_sum16(Gb[j][1] * G[j][0]);
        K[j][1][1] = row_sum16(Gb[j][1] * G[j][1]);
        if (mode == 2 && seg == p.nseg - 1) {
            // share of the final-angle gradient: <dh_final, J h_final>, h_final = Rot(Theta_final) g
            float s0 = 0.f, c0 = 1.f;
            if (piv(j) && i < NR) fast_sincos((float)wrap_2pi((double)p.thfin[bh * N2 + i]), s0, c0);
            float a = 0.f, bq = 0.f;
            if (piv(j) && cv && p.dh1) {
                a = p.dh1[(bh * N + 2 * i) * P + pc];
                bq = p.dh1[(bh * N + 2 * i + 1) * P + pc];
            }
            const float hf0 = c0 * G[j][0] - s0 * G[j][1], hf1 = s0 * G[j][0] + c0 * G[j][1];
            const float tj = row_sum16(-a * hf1 + bq * hf0);
            if (cc == 0 && piv(j)) p.thfp[(bh * p.ncg + cg) * N2 + i] = i < NR ? tj : 0.f;
        }
    }
    if (mode == 2) {
        __syncthreads();
        for (int e = tid; e < R * kCW; e += 256) sm[L::SPN + e] = 0.f;
    }
    float dDacc = 0.f;
    for (int blk = nblk - 1; blk >= 0; --blk) {
        const int64_t t0 = ts + (int64_t)blk * TBt;
        const int Tv = (int)min((int64_t)TBt, te - t0);
        __syncthreads();
        stage<Io, NPAD>(p, sm, b, h, cg, t0, Tv, true, mode == 2);
        __syncthreads();
        for (int k = Tv - 1; k >= 0; --k) {
            const float al = sm[L::SSC + k * 8 + 0], be = sm[L::SSC + k * 8 + 1], ga = sm[L::SSC + k * 8 + 2];
            if (mode == 1) {
#pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const int i = i0 + j;
                    if (!piv(j)) continue;
                    const float c = CS(k, i, 0), s = CS(k, i, 1);
                    float g0 = Gb[j][0], g1 = Gb[j][1];
#pragma unroll
                    for (int r = 0; r < RMAX; ++r) {
                        if (r >= R) break;
                        const int q_ = k * R + r;
                        const float yv = sm[L::SY + q_ * kCW + cc];
                        g0 += sm[L::SC + q_ * NPAD + 2 * i] * yv;
                        g1 += sm[L::SC + q_ * NPAD + 2 * i + 1] * yv;
                    }
                    Gb[j][0] = al * (c * g0 - s * g1);
                    Gb[j][1] = al * (s * g0 + c * g1);
                }
                continue;
            }
            float sq = 0.f, sbe = 0.f, sga = 0.f;
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                const int i = i0 + j;
                const bool iv = piv(j);
                const float c = iv ? CS(k, i, 0) : 1.f, s = iv ? CS(k, i, 1) : 0.f;
                float K00 = K[j][0][0], K01 = K[j][0][1], K10 = K[j][1][0], K11 = K[j][1][1];
#pragma unroll
                for (int r = 0; r < RMAX; ++r) {
                    if (r >= R) break;
                    const int q_ = k * R + r;
                    const float c0 = iv ? sm[L::SC + q_ * NPAD + 2 * i] : 0.f, c1 = iv ? sm[L::SC + q_ * NPAD + 2 * i + 1] : 0.f;
                    const float d0 = iv ? sm[L::SCB + q_ * NPAD + 2 * i] : 0.f, d1 = iv ? sm[L::SCB + q_ * NPAD + 2 * i + 1] : 0.f;
                    K00 += c0 * d0;
                    K01 += c0 * d1;
                    K10 += c1 * d0;
                    K11 += c1 * d1;
                    const float yv = sm[L::SY + q_ * kCW + cc];
                    Gb[j][0] += c0 * yv;
                    Gb[j][1] += c1 * yv;
                }
                float F00 = K00, F01 = K01, F10 = K10, F11 = K11;
                float V00 = 0.f, V01 = 0.f, V10 = 0.f, V11 = 0.f;
#pragma unroll
                for (int r = 0; r < RMAX; ++r) {
                    if (r >= R) break;
                    const float xc = SX(R + k * R + r), xp = SX(k * R + r);
                    const float u0 = row_sum16(Gb[j][0] * xc), u1 = row_sum16(Gb[j][1] * xc);
                    const float v0 = row_sum16(Gb[j][0] * xp), v1 = row_sum16(Gb[j][1] * xp);
                    const float b0 = iv ? SB(R + k * R + r, 2 * i) : 0.f, b1 = iv ? SB(R + k * R + r, 2 * i + 1) : 0.f;
                    const float p0 = iv ? SB(k * R + r, 2 * i) : 0.f, p1 = iv ? SB(k * R + r, 2 * i + 1) : 0.f;
                    F00 -= ga * u0 * b0;
                    F01 -= ga * u0 * b1;
                    F10 -= ga * u1 * b0;
                    F11 -= ga * u1 * b1;
                    V00 += v0 * p0;
                    V01 += v0 * p1;
                    V10 += v1 * p0;
                    V11 += v1 * p1;
                    const float qv0 = c * v0 - s * v1, qv1 = s * v0 + c * v1;  // Q^T v
                    sga += b0 * u0 + b1 * u1;
                    sbe += p0 * qv0 + p1 * qv1;
                    float nb0 = 0.f, nb1 = 0.f;
#pragma unroll
                    for (int rr = 0; rr < RMAX; ++rr)
                        if (rr == r) { nb0 = bpend[rr][j][0]; nb1 = bpend[rr][j][1]; }
                    if (cc == 0 && iv) {
                        const int64_t t = t0 + k;
                        float *dst = p.bbar + ((cg * BH + bh) * T + t) * (int64_t)N * R;
                        dst[(2 * i) * R + r] = nb0 + ga * u0;
                        dst[(2 * i + 1) * R + r] = nb1 + ga * u1;
                    }
#pragma unroll
                    for (int rr = 0; rr < RMAX; ++rr)
                        if (rr == r) { bpend[rr][j][0] = be * qv0; bpend[rr][j][1] = be * qv1; }
                }
                if (cc == 0 && iv && i < NR) p.tbar[((cg * BH + bh) * T + t0 + k) * (int64_t)N2 + i] = F01 - F10;
                const float E00 = F00 * c - F01 * s - be * V00, E01 = F00 * s + F01 * c - be * V01;
                const float E10 = F10 * c - F11 * s - be * V10, E11 = F10 * s + F11 * c - be * V11;
                sq += c * E00 + s * E01 - s * E10 + c * E11;
                K[j][0][0] = c * E00 - s * E10;
                K[j][0][1] = c * E01 - s * E11;
                K[j][1][0] = s * E00 + c * E10;
                K[j][1][1] = s * E01 + c * E11;
            }
            // dx partials: gamma part for token t, beta part for token t-1 (this lane's pairs)
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
                if (r >= R) break;
                const int q_ = k * R + r;
                float xg = 0.f, xb = 0.f;
#pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const int i = i0 + j;
                    if (!piv(j)) continue;
                    const float c = CS(k, i, 0), s = CS(k, i, 1);
                    const float b0 = SB(R + q_, 2 * i), b1 = SB(R + q_, 2 * i + 1);
                    const float p0 = SB(q_, 2 * i), p1 = SB(q_, 2 * i + 1);
                    const float qp0 = c * p0 + s * p1, qp1 = -s * p0 + c * p1;  // Q bprev
                    xg += b0 * Gb[j][0] + b1 * Gb[j][1];
                    xb += qp0 * Gb[j][0] + qp1 * Gb[j][1];
                }
                xg = rows_sum4(xg);
                xb = rows_sum4(xb);
                if (rho == 0) {
                    sm[L::SXG + (w * kRows + q_) * kCW + cc] = ga * xg;
                    sm[L::SXB + (w * kRows + q_) * kCW + cc] = be * xb;
                }
            }
            sq = rows_sum4(cc == 0 ? sq : 0.f);
            sbe = rows_sum4(cc == 0 ? sbe : 0.f);
            sga = rows_sum4(cc == 0 ? sga : 0.f);
            if (lane == 0) {
                sm[L::SSP + (k * 4 + w) * 4 + 0] = sq;
                sm[L::SSP + (k * 4 + w) * 4 + 1] = sbe;
                sm[L::SSP + (k * 4 + w) * 4 + 2] = sga;
            }
            // carry: G <- alpha Q^T G
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                const int i = i0 + j;
                if (!piv(j)) continue;
                const float c = CS(k, i, 0), s = CS(k, i, 1);
                const float g0 = Gb[j][0], g1 = Gb[j][1];
                Gb[j][0] = al * (c * g0 - s * g1);
                Gb[j][1] = al * (s * g0 + c * g1);
            }
        }
        if (mode == 1) continue;
        __syncthreads();
        // token scalars (this group's shares)
        if (tid < Tv * 3) {
            const int k = tid / 3, which = tid - 3 * k;
            float v = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) v += sm[L::SSP + (k * 4 + ww) * 4 + which];
            p.sbar[((cg * BH + bh) * T + t0 + k) * 4 + which] = v;
        }
        // dx of the group's columns: D dy + gamma part + beta part of the next token; a
        // segment's last token also gets the next segment's share, added by the final kernel
        for (int e = tid; e < Tv * R * kCW; e += 256) {
            const int q_ = e / kCW, c2 = e - q_ * kCW;
            const int k = q_ / R, r = q_ - k * R;
            const int col = cg * kCW + c2;
            const float yv = sm[L::SY + q_ * kCW + c2];
            float v = p.D[h] * yv;
            dDacc += yv * sm[L::SX + (R + q_) * kCW + c2];
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) v += sm[L::SXG + (ww * kRows + q_) * kCW + c2];
            const bool last_blk = blk == nblk - 1;
            if (k + 1 < Tv) {
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) v += sm[L::SXB + (ww * kRows + q_ + R) * kCW + c2];
            } else if (!last_blk) {
                v += sm[L::SPN + r * kCW + c2];
            }
            if (col >= P) continue;
            if (k + 1 == Tv && last_blk) {
                p.xlast[(sidx * R + r) * kCW + c2] = v;
            } else if (p.dx) {
                Io::st((ET *)p.dx + ((b * T + t0 + k) * H + h) * P * R + (int64_t)col * R + r, v);
            }
        }
        __syncthreads();
        // beta part produced at this block's first token: for the previous block's last token
        for (int e = tid; e < R * kCW; e += 256) {
            float v = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) v += sm[L::SXB + (ww * kRows + e / kCW) * kCW + e % kCW];
            sm[L::SPN + e] = v;
        }
    }
    if (mode == 1) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int i = i0 + j;
            if (!piv(j)) continue;
            p.Ragg[(sidx * N + 2 * i) * kCW + cc] = Gb[j][0];
            p.Ragg[(sidx * N + 2 * i + 1) * kCW + cc] = Gb[j][1];
        }
        return;
    }
    __syncthreads();
    // shares of the token before the segment: db (per pair, rank), dx (per column, rank)
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int i = i0 + j;
        if (!piv(j) || cc != 0) continue;
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
            if (r >= R) break;
            p.bpend[(sidx * N + 2 * i) * R + r] = bpend[r][j][0];
            p.bpend[(sidx * N + 2 * i + 1) * R + r] = bpend[r][j][1];
        }
    }
    for (int e = tid; e < R * kCW; e += 256) p.xpend[sidx * R * kCW + e] = sm[L::SPN + e];
    // D gradient share
    dDacc = wave_sum(dDacc);
    if (lane == 0) sm[L::SRD + w] = dDacc;
    __syncthreads();
    if (tid == 0) p.dDp[sidx] = sm[L::SRD] + sm[L::SRD + 1] + sm[L::SRD + 2] + sm[L::SRD + 3];
}

// Segment start states from the forward aggregates (in place), and the final angle.
// One thread per (sequence, column group, pair).
__global__ __launch_bounds__(256) void bwd_ffold_kernel(BwdParams p) {
    const int N = p.N, N2 = N / 2, P = p.P, NR = p.nr;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= p.B * p.H * p.ncg * N2) return;
    const int i = (int)(e % N2);
    const int64_t q = e / N2;
    const int cg = (int)(q % p.ncg);
    const int64_t bh = q / p.ncg;
    float s0 = 0.f, c0 = 1.f;
    double th = 0.0;
    if (p.ang0 && i < NR) {
        th = (double)p.ang0[bh * NR + i];
        fast_sincos((float)wrap_2pi(th), s0, c0);
    }
    float g[kCW][2];
#pragma unroll
    for (int c = 0; c < kCW; ++c) {
        const int pc = cg * kCW + c;
        float u = 0.f, v = 0.f;
        if (p.h0 && pc < P) {
            u = p.h0[(bh * N + 2 * i) * P + pc];
            v = p.h0[(bh * N + 2 * i + 1) * P + pc];
        }
        g[c][0] = c0 * u + s0 * v;
        g[c][1] = -s0 * u + c0 * v;
    }
    for (int k = 0; k < p.nseg; ++k) {
        const int64_t sidx = (bh * p.ncg + cg) * p.nseg + k;
        const float dec = __expf(p.lseg[bh * p.nseg + k]);
        const float ang = p.pseg[(bh * p.nseg + k) * N2 + i];
        th += (double)ang;
        float s, c;
        fast_sincos((float)wrap_2pi((double)ang), s, c);
        float *ga = p.Gagg + (sidx * N + 2 * i) * kCW;
#pragma unroll
        for (int cc = 0; cc < kCW; ++cc) {
            const float a0 = ga[cc], a1 = ga[kCW + cc];
            ga[cc] = g[cc][0];
            ga[kCW + cc] = g[cc][1];
            const float u = dec * g[cc][0], v = dec * g[cc][1];
            g[cc][0] = c * u + s * v + a0;  // Rot(-phi)
            g[cc][1] = -s * u + c * v + a1;
        }
    }
    if (cg == 0) p.thfin[bh * N2 + i] = i < NR ? (float)wrap_2pi(th) : 0.f;
}

// Segment end adjoints from the adjoint aggregates (in place), the gradient of the
// initial h and the initial-angle share from it.  One thread per (sequence, group, pair).
__global__ __launch_bounds__(256) void bwd_rfold_kernel(BwdParams p) {
    const int N = p.N, N2 = N / 2, P = p.P, NR = p.nr;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= p.B * p.H * p.ncg * N2) return;
    const int i = (int)(e % N2);
    const int64_t q = e / N2;
    const int cg = (int)(q % p.ncg);
    const int64_t bh = q / p.ncg;
    float s0 = 0.f, c0 = 1.f;
    if (i < NR) fast_sincos(p.thfin[bh * N2 + i], s0, c0);
    float a[kCW][2];
#pragma unroll
    for (int c = 0; c < kCW; ++c) {
        const int pc = cg * kCW + c;
        float u = 0.f, v = 0.f;
        if (p.dh1 && pc < P) {
            u = p.dh1[(bh * N + 2 * i) * P + pc];
            v = p.dh1[(bh * N + 2 * i + 1) * P + pc];
        }
        a[c][0] = c0 * u + s0 * v;  // Rot(-Theta_final) dh_final
        a[c][1] = -s0 * u + c0 * v;
    }
    for (int k = p.nseg - 1; k >= 0; --k) {
        const int64_t sidx = (bh * p.ncg + cg) * p.nseg + k;
        const float dec = __expf(p.lseg[bh * p.nseg + k]);
        float s, c;
        fast_sincos((float)wrap_2pi((double)p.pseg[(bh * p.nseg + k) * N2 + i]), s, c);
        float *ra = p.Ragg + (sidx * N + 2 * i) * kCW;
#pragma unroll
        for (int cc = 0; cc < kCW; ++cc) {
            const float r0 = ra[cc], r1 = ra[kCW + cc];
            ra[cc] = a[cc][0];
            ra[kCW + cc] = a[cc][1];
            const float u = dec * a[cc][0], v = dec * a[cc][1];
            a[cc][0] = c * u - s * v + r0;  // Rot(+phi)
            a[cc][1] = s * u + c * v + r1;
        }
    }
    // gradient of g_{-1} -> dh0 = Rot(Theta_init) a ; initial-angle share <a, -J g_{-1}>
    float si = 0.f, ci = 1.f;
    if (p.ang0 && i < NR) fast_sincos((float)wrap_2pi((double)p.ang0[bh * NR + i]), si, ci);
    float ta = 0.f;
#pragma unroll
    for (int c = 0; c < kCW; ++c) {
        const int pc = cg * kCW + c;
        if (pc >= P) continue;
        if (p.dh0) {
            p.dh0[(bh * N + 2 * i) * P + pc] = ci * a[c][0] - si * a[c][1];
            p.dh0[(bh * N + 2 * i + 1) * P + pc] = si * a[c][0] + ci * a[c][1];
        }
        if (p.h0) {
            const float u = p.h0[(bh * N + 2 * i) * P + pc], v = p.h0[(bh * N + 2 * i + 1) * P + pc];
            const float g0 = ci * u + si * v, g1 = -si * u + ci * v;
            ta += a[c][0] * g1 - a[c][1] * g0;
        }
    }
    p.dang0p[(bh * p.ncg + cg) * N2 + i] = ta;
}

// Per-token sums of the column-group shares, the boundary terms, the norm backward
// of B and C, and the initial state's remaining gradients.  Grid (sequence, 16-token
// block); one wave per (token, rank) row in the norm backward.
template <class Io>
__global__ __launch_bounds__(256) void bwd_final_kernel(BwdParams p) {
    using ET = typename Io::T;
    __shared__ float s_thf[64];        // total final-angle gradient of the sequence, per pair
    __shared__ float s_bl[8][128];     // b of the last token (complex form), per rank
    __shared__ float s_acc[4][3];
    __shared__ float s_bias[4 * 2 * 8 * 128];  // per wave, side, rank, n
    const int N = p.N, N2 = N / 2, P = p.P, R = p.R, NR = p.nr;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int tb = blockIdx.y;
    const int64_t b = bh / p.H;
    const int h = (int)(bh - b * p.H);
    const int64_t T = p.T, H = p.H, BH = p.B * p.H;
    const int ncg = p.ncg;
    // b of the last token, then the final-angle gradient
    for (int r = w; r < R; r += 4) {
        const int64_t bth = (b * T + T - 1) * H + h;
        norm_row<Io>(p, (const ET *)p.Bm + bth * N * R + r, R, p.bnw,
                     p.bbias ? p.bbias + ((int64_t)h * R + r) * N : nullptr, s_bl[r]);
    }
    __syncthreads();
    if (tid < N2) {
        const int i = tid;
        float v = 0.f;
        if (i < NR) {
            for (int cg = 0; cg < ncg; ++cg) v += p.thfp[(bh * ncg + cg) * N2 + i];
            if (p.dang1) v += p.dang1[bh * NR + i];
            float s0, c0;
            fast_sincos(p.thfin[bh * N2 + i], s0, c0);
            if (p.dpB1)
                for (int r = 0; r < R; ++r) {
                    const float u = s_bl[r][2 * i], vv = s_bl[r][2 * i + 1];
                    const float pb0 = c0 * u - s0 * vv, pb1 = s0 * u + c0 * vv;  // prev_B of the final state
                    v += -p.dpB1[(bh * N + 2 * i) * R + r] * pb1 + p.dpB1[(bh * N + 2 * i + 1) * R + r] * pb0;
                }
        }
        s_thf[i] = v;
    }
    __syncthreads();
    float aA = 0.f, aDtb = 0.f;
    float gB[2] = {0.f, 0.f}, gC[2] = {0.f, 0.f};
    float *part = p.part + (bh * p.ntb + tb) * (int64_t)p.pw;
    const int64_t t0 = (int64_t)tb * 16;
    const int Tv = (int)min((int64_t)16, T - t0);
    // token scalars
    if (tid < Tv) {
        const int64_t t = t0 + tid;
        const int64_t bth = (b * T + t) * H + h;
        float qv = 0.f, bb = 0.f, gb = 0.f;
        for (int cg = 0; cg < ncg; ++cg) {
            const float *s = p.sbar + ((cg * BH + bh) * T + t) * 4;
            qv += s[0];
            bb += s[1];
            gb += s[2];
        }
        float dt, lam, dsp, dsg;
        act_scalars(p, bth, h, dt, lam, dsp, dsg);
        const float A = (p.flags & kFlagAPerToken) ? p.A[bth] : p.A[h];
        const float al = __expf(dt * A), be = al * dt * (1.f - lam);
        float ddt = qv * A + bb * al * (1.f - lam) * (1.f + dt * A) + gb * lam;
        float dlm = -bb * al * dt + gb * dt;
        const float dAv = qv * dt + bb * be * dt;
        ddt *= dsp;
        dlm *= dsg;
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
            const int64_t t = t0 + k;
            float v = s_thf[i];
            for (int cg = 0; cg < ncg; ++cg) v += p.tbar[((cg * BH + bh) * T + t) * (int64_t)N2 + i];
            p.dtheta[((b * T + t) * H + h) * (int64_t)NR + i] = v;
        }
    // dx of segment-last tokens: the segment's own part and the next segment's share
    for (int e = tid; e < Tv * R * P; e += 256) {
        const int k = e / (R * P), rem = e - k * R * P, r = rem / P, pc = rem - r * P;
        const int64_t t = t0 + k;
        if ((t + 1) % p.segT != 0 && t != T - 1) continue;
        const int seg = (int)(t / p.segT), cg = pc / kCW, c2 = pc - cg * kCW;
        const int64_t sidx = (bh * ncg + cg) * p.nseg + seg;
        float v = p.xlast[(sidx * R + r) * kCW + c2];
        if (t == T - 1) {
            if (p.dpx1) v += p.dpx1[(bh * P + pc) * R + r];
        } else {
            v += p.xpend[((sidx + 1) * R + r) * kCW + c2];
        }
        if (p.dx) Io::st((ET *)p.dx + ((b * T + t) * H + h) * P * R + (int64_t)pc * R + r, v);
    }
    // db and dc rows: sums of the shares (plus the boundary shares of db), norm backward;
    // rows spread over the waves, bias gradients collected per wave in LDS
    for (int e = tid; e < 4 * 2 * R * N; e += 256) s_bias[e] = 0.f;
    __syncthreads();
    for (int q = w; q < Tv * R; q += 4) {
        const int k = q / R, r = q - k * R;
        const int64_t t = t0 + k;
        const int64_t bth = (b * T + t) * H + h;
        const int seg = (int)(t / p.segT);
        const bool segl = (t + 1) % p.segT == 0 && t != T - 1;
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            const ET *raw = (const ET *)(side == 0 ? p.Bm : p.Cm) + bth * N * R + r;
            const float *gain = side == 0 ? p.bnw : p.cnw;
            const float *src = side == 0 ? p.bbar : p.cbar;
            const bool norm = (p.flags & kFlagNorm) != 0;
            float v[2], gv[2], ss = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int n = lane + 64 * kk;
                v[kk] = n < N ? Io::ld(raw + (int64_t)n * R) : 0.f;
                ss += v[kk] * v[kk];
                float g = 0.f;
                if (n < N) {
                    for (int cg = 0; cg < ncg; ++cg) g += src[((cg * BH + bh) * T + t) * (int64_t)N * R + n * R + r];
                    if (side == 0 && segl)
                        for (int cg = 0; cg < ncg; ++cg)
                            g += p.bpend[(((bh * ncg + cg) * p.nseg + seg + 1) * N + n) * R + r];
                    if (side == 0 && t == T - 1 && p.dpB1) {
                        // prev_B of the final state is Rot(Theta_final) b_{T-1}
                        const int i = n >> 1;
                        float s0 = 0.f, c0 = 1.f;
                        if (i < NR) fast_sincos(p.thfin[bh * N2 + i], s0, c0);
                        const float d0 = p.dpB1[(bh * N + 2 * i) * R + r], d1 = p.dpB1[(bh * N + 2 * i + 1) * R + r];
                        g += (n & 1) ? (-s0 * d0 + c0 * d1) : (c0 * d0 + s0 * d1);
                    }
                }
                gv[kk] = g;
            }
            ss = wave_sum(ss);
            const float rs = norm ? rsqrtf(ss / (float)N + p.eps) : 1.f;
            float dot = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int n = lane + 64 * kk;
                const float gn = (n < N && gain) ? gain[n] : 1.f;
                dot += gv[kk] * gn * v[kk];
                if (n < N) s_bias[((w * 2 + side) * R + r) * N + n] += gv[kk];
                if (norm) (side == 0 ? gB : gC)[kk] += gv[kk] * v[kk] * rs;
            }
            dot = wave_sum(dot);
            ET *out = (ET *)(side == 0 ? p.dB : p.dC);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int n = lane + 64 * kk;
                if (n >= N || !out) continue;
                const float gn = gain ? gain[n] : 1.f;
                const float d = norm ? gv[kk] * gn * rs - dot * rs * rs * rs * v[kk] / (float)N : gv[kk];
                Io::st(out + bth * N * R + (int64_t)n * R + r, d);
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < 2 * R * N; e += 256) {
        const int side = e / (R * N), rn = e - side * R * N;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) v += s_bias[(ww * 2 + side) * R * N + rn];
        part[3 + 2 * N + side * R * N + rn] = v;
    }
    // the initial state's prev_B, prev_x and angle gradients (first token block only)
    if (tb == 0) {
        for (int e = tid; e < N2 * R; e += 256) {
            const int i = e / R, r = e - i * R;
            float d0 = 0.f, d1 = 0.f;
            for (int cg = 0; cg < ncg; ++cg) {
                const int64_t sidx = (bh * ncg + cg) * p.nseg;
                d0 += p.bpend[(sidx * N + 2 * i) * R + r];
                d1 += p.bpend[(sidx * N + 2 * i + 1) * R + r];
            }
            float si = 0.f, ci = 1.f;
            if (p.ang0 && i < NR) fast_sincos((float)wrap_2pi((double)p.ang0[bh * NR + i]), si, ci);
            if (p.dpB0) {
                p.dpB0[(bh * N + 2 * i) * R + r] = ci * d0 - si * d1;
                p.dpB0[(bh * N + 2 * i + 1) * R + r] = si * d0 + ci * d1;
            }
        }
        if (p.dpx0)
            for (int e = tid; e < P * R; e += 256) {
                const int pc = e / R, r = e - pc * R, cg = pc / kCW;
                p.dpx0[(bh * P + pc) * R + r] = p.xpend[(((bh * ncg + cg) * p.nseg) * R + r) * kCW + pc % kCW];
            }
        if (p.dang0 && tid < NR) {
            const int i = tid;
            float v = s_thf[i];
            for (int cg = 0; cg < ncg; ++cg) v += p.dang0p[(bh * ncg + cg) * N2 + i];
            for (int r = 0; r < R; ++r) {
                float d0 = 0.f, d1 = 0.f;
                for (int cg = 0; cg < ncg; ++cg) {
                    const int64_t sidx = (bh * ncg + cg) * p.nseg;
                    d0 += p.bpend[(sidx * N + 2 * i) * R + r];
                    d1 += p.bpend[(sidx * N + 2 * i + 1) * R + r];
                }
                float u, vv;
                init_b(p, bh, i, r, u, vv);
                v += d0 * vv - d1 * u;
            }
            p.dang0[bh * NR + i] = v;
        }
    }
    // parameter partials of this block
    {
        const float v1 = wave_sum(aA), v2 = wave_sum(aDtb);
        if (lane == 0) {
            s_acc[w][0] = v1;
            s_acc[w][1] = v2;
        }
    }
    __syncthreads();
    if (tid == 0) {
        part[0] = s_acc[0][0] + s_acc[1][0] + s_acc[2][0] + s_acc[3][0];
        part[2] = s_acc[0][1] + s_acc[1][1] + s_acc[2][1] + s_acc[3][1];
        part[1] = 0.f;  // D is summed from the sweep shares
    }
    __syncthreads();
    // gains: per-wave sums through LDS
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int n = lane + 64 * kk;
        if (n < N) {
            s_bias[(w * 2 + 0) * N + n] = gB[kk];
            s_bias[(w * 2 + 1) * N + n] = gC[kk];
        }
    }
    __syncthreads();
    for (int e = tid; e < 2 * N; e += 256) {
        const int side = e / N, n = e - side * N;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) v += s_bias[(ww * 2 + side) * N + n];
        part[3 + side * N + n] = v;
    }
}

// Parameter gradients: one workgroup per parameter element sums its records (the final
// kernel's per (sequence, token block) records, the sweeps' D shares) in a fixed order.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p) {
    __shared__ float s_red[256];
    const int H = p.H, N = p.N, R = p.R;
    const int64_t Bn = p.B;
    const int e = blockIdx.x, tid = threadIdx.x;
    const int nH = 3 * H, nG = 2 * N;
    const int ntb = p.ntb;
    float *dst = nullptr;
    float v = 0.f;
    if (e < nH) {
        const int which = e / H, h = e - which * H;  // 0: A, 1: D, 2: dt bias
        dst = which == 0 ? p.dA : (which == 1 ? p.dD : p.ddtb);
        if (dst) dst += h;
        if (which == 1) {
            const int per = p.ncg * p.nseg;
            for (int64_t k = tid; k < Bn * per; k += 256) {
                const int64_t b = k / per;
                v += p.dDp[(b * H + h) * (int64_t)per + (k - b * per)];
            }
        } else {
            for (int64_t k = tid; k < Bn * ntb; k += 256) {
                const int64_t b = k / ntb;
                v += p.part[((b * H + h) * ntb + (k - b * ntb)) * (int64_t)p.pw + which];
            }
        }
    } else if (e < nH + nG) {
        const int k2 = e - nH, side = k2 / N, n = k2 - side * N;
        dst = side == 0 ? p.dbnw : p.dcnw;
        if (dst) dst += n;
        for (int64_t s = tid; s < Bn * H * ntb; s += 256) v += p.part[s * p.pw + 3 + side * N + n];
    } else {
        const int k2 = e - nH - nG, side = k2 / (H * R * N), rem = k2 - side * (H * R * N);
        const int h = rem / (R * N), rn = rem - h * (R * N);
        dst = side == 0 ? p.dbb : p.dcb;
        if (dst) dst += rem;
        for (int64_t k = tid; k < Bn * ntb; k += 256) {
            const int64_t b = k / ntb;
            v += p.part[((b * H + h) * ntb + (k - b * ntb)) * (int64_t)p.pw + 3 + 2 * N + side * R * N + rn];
        }
    }
    if (!dst) return;  // uniform over the workgroup
    s_red[tid] = v;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if (tid < st) s_red[tid] += s_red[tid + st];
        __syncthreads();
    }
    if (tid == 0) *dst = s_red[0];
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
        if (p.dA) p.dA[e] = 0.f;
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

template <class Io, int NPAD>
static void launch_sweeps(const BwdParams &p, hipStream_t st, int mode) {
    const dim3 grid((unsigned)(p.B * p.H * p.ncg * p.nseg)), blk(256);
    if (p.R == 1) hipLaunchKernelGGL((bwd_sweep_kernel<Io, NPAD, 1>), grid, blk, 0, st, p, mode);
    else hipLaunchKernelGGL((bwd_sweep_kernel<Io, NPAD, 8>), grid, blk, 0, st, p, mode);
}

template <class Io>
static hipError_t launch_bwd_t(const BwdParams &p, hipStream_t st) {
    const int npad = p.N <= 32 ? 32 : (p.N <= 64 ? 64 : 128);
    auto sweep = [&](int mode) {
        if (npad == 32) launch_sweeps<Io, 32>(p, st, mode);
        else if (npad == 64) launch_sweeps<Io, 64>(p, st, mode);
        else launch_sweeps<Io, 128>(p, st, mode);
    };
    const int64_t nfold = p.B * p.H * p.ncg * (p.N / 2);
    const dim3 fgrid((unsigned)((nfold + 255) / 256));
    sweep(0);
    hipLaunchKernelGGL(bwd_ffold_kernel, fgrid, dim3(256), 0, st, p);
    sweep(1);
    hipLaunchKernelGGL(bwd_rfold_kernel, fgrid, dim3(256), 0, st, p);
    sweep(2);
    hipLaunchKernelGGL((bwd_final_kernel<Io>), dim3((unsigned)(p.B * p.H), (unsigned)p.ntb), dim3(256), 0, st, p);
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
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)total), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace m3
