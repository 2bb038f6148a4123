// m3_chunk.hip -- chunk kernels of the chunked Mamba-3 scan on gfx950.
//
// Chunkwise SSD (torchmamba README, "Math notes", M2: an intra-chunk
// quadratic part plus a factored state carry between chunks) applied to the
// Mamba-3 trapezoid in its single-scan form (dotLLM PR #136, comment
// "Mamba-3 streaming decode": per-token scale gamma_t + eta_t with the
// one-token lookahead eta_t = dt_{t+1}(1 - lambda_{t+1}), which must cross
// chunk edges).  With the shifted state h'_t = h_t + eta_t B~_t x_t^T:
//     h'_t = alpha_t h'_{t-1} + (gamma_t + eta_t) B~_t x_t^T
//     y_t  = C~_t^T h'_t - eta_t (C~_t . B~_t) x_t + D x_t
// so inside a chunk the mask is
//     L[t, s] = exp(cs_t - cs_s) * (s < t ? scale_s : s == t ? gamma_t : 0),
// cs = running sum of dt*A inside the chunk.  Rotations use chunk-local
// angles (running sum of theta from the chunk start); the carried state is
// kept in the frame of the chunk it enters.
//
// One workgroup (4 waves) per (chunk, head, batch).  Rows of a chunk are
// (token, rank) pairs, rank fastest (SISO: rows = tokens).
//   MODE_STATE : S^T[p][n] = sum_s x_s[p] w_s B~_s[n],  w_s = exp(cs_end - cs_s) scale_s,
//                plus the chunk decay exp(cs_end) and angle totals.
//   MODE_OUTPUT: y = (L o C~ B~^T) X + exp(cs_t) C~ H_c + D x with H_c from the state pass.
// Operands: bf16 I/O uses bf16 MFMA with every non-exact operand split into
// hi + lo bf16 (three products); fp32 I/O uses the fp32 MFMA.
#include <type_traits>

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

template <class Io, int ROWS, int NP, int PP, int MODE>
struct ChunkCfg {
    static constexpr bool BF = std::is_same<Io, IoBF16>::value;
    static constexpr int NRT = ROWS / 16;  // row tiles
    static constexpr int KS = NP / 32;     // 32-wide k steps over n
    static constexpr int PT = PP / 16;     // p tiles
    static constexpr int NT = NP / 16;     // n tiles
    static constexpr int RTW = (NRT + 3) / 4;  // row tiles per wave
    static constexpr int ES = BF ? 2 : 4;      // bytes per operand element per plane
    static constexpr int NPL = BF ? 2 : 1;     // planes (hi, lo) or (fp32)
    static constexpr int PADE = BF ? 8 : 4;    // 16 bytes of padding per row
    static constexpr int OPP = NP + PADE;      // pitch of [row][n] and [p][n] planes
    static constexpr int RPP = ROWS + PADE;    // pitch of [p][row] and [n][row] planes
    static constexpr int PHP = NP / 2;         // pitch of the angle table [token][pair]
    // region 0: B~ [row][n] (output mode) or w*B~^T [n][row] (state mode); later the y staging
    static constexpr size_t OP_PLANE = (MODE == MODE_OUTPUT) ? (size_t)ROWS * OPP : (size_t)NP * RPP;
    static constexpr size_t R0_OP = OP_PLANE * ES * NPL;
    static constexpr size_t R0_Y = (MODE == MODE_OUTPUT) ? (size_t)ROWS * PP * sizeof(typename Io::T) : 0;
    static constexpr size_t R0 = ((R0_OP > R0_Y ? R0_OP : R0_Y) + 15) / 16 * 16;
    // region 1: X^T [p][row]  (bf16 exact or fp32)
    static constexpr size_t R1 = ((size_t)PP * RPP * ES + 15) / 16 * 16;
    // region 2: angle table [token][pair]; in output mode later H^T [p][n] planes
    static constexpr size_t R2_PHI = (size_t)ROWS * PHP * 4;
    static constexpr size_t H_PLANE = (size_t)PP * OPP;
    static constexpr size_t R2_H = (MODE == MODE_OUTPUT) ? H_PLANE * ES * NPL : 0;
    static constexpr size_t R2 = ((R2_PHI > R2_H ? R2_PHI : R2_H) + 15) / 16 * 16;
    // region 3: per-token scalars (cs, scale, gamma, w, exp(cs)) + scan scratch (256 floats)
    static constexpr size_t R3 = (size_t)(5 * ROWS + 256 + 64) * 4;
    static constexpr size_t BYTES = R0 + R1 + R2 + R3;
};

// row tile owned by (wave, k): balanced pairing for 8 tiles (w, 7-w), else w + 4k
template <int NRT>
__device__ __forceinline__ int owned_tile(int wave, int k) {
    if (NRT == 8) return k == 0 ? wave : 7 - wave;
    return wave + 4 * k;
}

template <class Io, int ROWS, int NP, int PP, int MODE>
__global__ __launch_bounds__(256) void chunk_kernel(ScanParams p) {
    using Cfg = ChunkCfg<Io, ROWS, NP, PP, MODE>;
    using ET = typename Io::T;
    constexpr bool BF = Cfg::BF;
    constexpr int NRT = Cfg::NRT, KS = Cfg::KS, PT = Cfg::PT, NT = Cfg::NT, RTW = Cfg::RTW;
    constexpr int OPP = Cfg::OPP, RPP = Cfg::RPP, PHP = Cfg::PHP;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char *r0 = smem;
    unsigned char *r1 = smem + Cfg::R0;
    unsigned char *r2 = r1 + Cfg::R1;
    float *s_cs = (float *)(r2 + Cfg::R2);
    float *s_scale = s_cs + ROWS;
    float *s_gam = s_scale + ROWS;
    float *s_w = s_gam + ROWS;
    float *s_ecs = s_w + ROWS;
    float *s_tmp = s_ecs + ROWS;  // 256 + 64 floats of scan scratch
    float *s_phi = (float *)r2;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int c = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int R = p.R, N = p.N, P = p.P, N2 = p.N / 2, Q = p.Q;
    const int64_t T = p.T, H = p.H;
    const int64_t t0 = (int64_t)c * Q;
    const int Qv = (int)((T - t0) < (int64_t)Q ? (T - t0) : (int64_t)Q);  // valid tokens, >= 1
    const int Rv = Qv * R;                                                // valid rows
    const int64_t bh = b * H + h;
    const bool last_chunk = (c == p.nchunks - 1);
    const bool want_final = (MODE == MODE_OUTPUT) && last_chunk && (p.h1 != nullptr);

    // ---------------------------------------------------------- per-token scalars
    // tokens 0..ROWS-1 (only t < Qv are real; the rest get log alpha = gamma = scale = 0)
    float la = 0.f, ga = 0.f, sc = 0.f;
    if (tid < Qv) {
        const int64_t gi = (b * T + t0 + tid) * H + h;
        const float dtv = p.dt[gi], lmv = p.lam[gi];
        la = dtv * p.A[h];
        ga = lmv * dtv;
        float eta = 0.f;
        if (t0 + tid + 1 < T) {
            const int64_t gn = gi + H;
            eta = p.dt[gn] * (1.f - p.lam[gn]);
        }
        sc = ga + eta;
    }
    // inclusive scan of log alpha over tokens (<= 128: waves 0 and 1)
    float cs = la;
    if (tid < ROWS) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            float o = __shfl_up(cs, off, 64);
            if (lane >= off) cs += o;
        }
        if (lane == 63) s_tmp[256 + wave] = cs;
    }
    // angle table: theta of valid tokens
    for (int e = tid; e < Qv * N2; e += 256) {
        const int t = e / N2, i = e - t * N2;
        s_phi[t * PHP + i] = p.theta[((b * T + t0 + t) * H + h) * N2 + i];
    }
    __syncthreads();
    if (tid < ROWS) {
        if (wave == 1) cs += s_tmp[256 + 0];
        s_cs[tid] = cs;
        s_scale[tid] = sc;
        s_gam[tid] = ga;
        s_ecs[tid] = __expf(cs);
    }
    // running angle inside the chunk: segmented scan along tokens, per pair
    {
        int nseg = 256 / N2;
        if (nseg > Qv) nseg = Qv;
        if (nseg < 1) nseg = 1;
        const int seglen = (Qv + nseg - 1) / nseg;
        const int i = tid % N2, sg = tid / N2;
        float acc = 0.f;
        if (sg < nseg) {
            const int ta = sg * seglen, tb = min(Qv, ta + seglen);
            for (int t = ta; t < tb; ++t) {
                acc += s_phi[t * PHP + i];
                s_phi[t * PHP + i] = acc;
            }
            s_tmp[sg * N2 + i] = acc;
        }
        __syncthreads();
        if (sg < nseg && sg > 0) {
            float off = 0.f;
            for (int k = 0; k < sg; ++k) off += s_tmp[k * N2 + i];
            const int ta = sg * seglen, tb = min(Qv, ta + seglen);
            for (int t = ta; t < tb; ++t) s_phi[t * PHP + i] += off;
        }
    }
    __syncthreads();
    const float cs_end = s_cs[ROWS - 1];
    if (tid < ROWS) s_w[tid] = __expf(cs_end - s_cs[tid]) * s_scale[tid];
    __syncthreads();

    // ---------------------------------------------------------- X^T [p][row]
    {
        const ET *xg = (const ET *)p.x;
        for (int e = tid; e < ROWS * PP; e += 256) {
            const int row = e / PP, pc = e - row * PP;
            const int tok = row / R, r = row - tok * R;
            if (BF) {
                uint16_t v = 0;
                if (tok < Qv && pc < P) v = ((const uint16_t *)xg)[((b * T + t0 + tok) * H + h) * P * R + pc * R + r];
                ((uint16_t *)r1)[pc * RPP + row] = v;
            } else {
                float v = 0.f;
                if (tok < Qv && pc < P) v = ((const float *)xg)[((b * T + t0 + tok) * H + h) * P * R + pc * R + r];
                ((float *)r1)[pc * RPP + row] = v;
            }
        }
    }

    // ---------------------------------------------------------- B~ (and C~) rows
    typedef typename std::conditional<BF, FragHL, FragF>::type OpFrag;
    OpFrag ct[RTW][KS];  // C~ of the owned row tiles (output mode)
    const bool bcnorm = (p.flags & 1u) != 0;
    const float *thfin = p.thfin + bh * N2;
#pragma unroll
    for (int k = 0; k < RTW; ++k) {
        const int rt = owned_tile<NRT>(wave, k);
        if (rt >= NRT) continue;
        const int row = rt * 16 + l16;
        const int tok = row / R, r = row - tok * R;
        const bool rv = tok < Qv;
        const int64_t base = ((b * T + t0 + tok) * H + h) * (int64_t)N * R + r;
        float vb[KS][8], vc[KS][8];
        float ssb = 0.f, ssc = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int n = kk * 32 + 8 * g + j;
                const bool ok = rv && n < N;
                vb[kk][j] = ok ? Io::ld((const ET *)p.Bm + base + (int64_t)n * R) : 0.f;
                ssb += vb[kk][j] * vb[kk][j];
                if (MODE == MODE_OUTPUT) {
                    vc[kk][j] = ok ? Io::ld((const ET *)p.Cm + base + (int64_t)n * R) : 0.f;
                    ssc += vc[kk][j] * vc[kk][j];
                }
            }
        }
        ssb += __shfl_xor(ssb, 16, 64);
        ssb += __shfl_xor(ssb, 32, 64);
        ssc += __shfl_xor(ssc, 16, 64);
        ssc += __shfl_xor(ssc, 32, 64);
        const float rsb = bcnorm ? rsqrtf(ssb / (float)N + p.eps) : 1.f;
        const float rsc = bcnorm ? rsqrtf(ssc / (float)N + p.eps) : 1.f;
        const float wt = rv ? s_w[tok] : 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float ob[8], oc[8];
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) {
                const int n = kk * 32 + 8 * g + 2 * jp;
                float b0 = 0.f, b1 = 0.f, c0 = 0.f, c1 = 0.f;
                if (rv && n < N) {
                    float gb0 = 1.f, gb1 = 1.f, gc0 = 1.f, gc1 = 1.f;
                    if (bcnorm && p.bnw) { gb0 = p.bnw[n]; gb1 = p.bnw[n + 1]; }
                    if (bcnorm && p.cnw) { gc0 = p.cnw[n]; gc1 = p.cnw[n + 1]; }
                    float u = vb[kk][2 * jp] * rsb * gb0, w = vb[kk][2 * jp + 1] * rsb * gb1;
                    if (p.bbias) {
                        u += p.bbias[((int64_t)h * R + r) * N + n];
                        w += p.bbias[((int64_t)h * R + r) * N + n + 1];
                    }
                    float sn, cn;
                    sincosf(s_phi[tok * PHP + n / 2], &sn, &cn);
                    b0 = u * cn - w * sn;
                    b1 = u * sn + w * cn;
                    if (want_final && t0 + tok == T - 1) {
                        // carried B~ of the last token, in the global frame of the final angle
                        float s2, c2;
                        sincosf(thfin[n / 2], &s2, &c2);
                        p.pB1[(bh * N + n) * R + r] = u * c2 - w * s2;
                        p.pB1[(bh * N + n + 1) * R + r] = u * s2 + w * c2;
                    }
                    if (MODE == MODE_OUTPUT) {
                        float uc = vc[kk][2 * jp] * rsc * gc0, wc = vc[kk][2 * jp + 1] * rsc * gc1;
                        if (p.cbias) {
                            uc += p.cbias[((int64_t)h * R + r) * N + n];
                            wc += p.cbias[((int64_t)h * R + r) * N + n + 1];
                        }
                        c0 = uc * cn - wc * sn;
                        c1 = uc * sn + wc * cn;
                    }
                }
                ob[2 * jp] = b0;
                ob[2 * jp + 1] = b1;
                oc[2 * jp] = c0;
                oc[2 * jp + 1] = c1;
            }
            if (MODE == MODE_OUTPUT) {
                // B~ row -> [row][n] planes; C~ stays in registers
                const int off = row * OPP + kk * 32 + 8 * g;
                if constexpr (BF) {
                    FragHL f = make_hl(ob);
                    uint16_t *hi = (uint16_t *)r0;
                    *(u32x4_t *)(hi + off) = f.hi;
                    *(u32x4_t *)(hi + Cfg::OP_PLANE + off) = f.lo;
                    ct[k][kk] = make_hl(oc);
                } else {
                    float *fp = (float *)r0;
                    *(f32x4_t *)(fp + off) = f32x4_t{ob[0], ob[1], ob[2], ob[3]};
                    *(f32x4_t *)(fp + off + 4) = f32x4_t{ob[4], ob[5], ob[6], ob[7]};
                    ct[k][kk] = make_f(oc);
                }
            } else {
                // w * B~ -> transposed [n][row] planes
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int n = kk * 32 + 8 * g + j;
                    const float v = ob[j] * wt;
                    if constexpr (BF) {
                        uint32_t hi, lo;
                        split_hl(v, hi, lo);
                        ((uint16_t *)r0)[n * RPP + row] = (uint16_t)hi;
                        ((uint16_t *)r0)[Cfg::OP_PLANE + n * RPP + row] = (uint16_t)lo;
                    } else {
                        ((float *)r0)[n * RPP + row] = v;
                    }
                }
            }
        }
    }

    if (MODE == MODE_STATE) {
        __syncthreads();
        // chunk totals: decay and angle
        const int64_t bhc = bh * p.nchunks + c;
        if (tid == 0) p.decay[bhc] = s_ecs[Qv - 1];
        if (tid < N2) {
            const float ph = s_phi[(Qv - 1) * PHP + tid];
            float sn, cn;
            sincosf(ph, &sn, &cn);
            p.phi[bhc * N2 + tid] = ph;
            p.cphi[bhc * N2 + tid] = cn;
            p.sphi[bhc * N2 + tid] = sn;
        }
        // S^T[p][n] = X^T (w B~): A = X^T [p][row], B = (w B~)^T [n][row]
        float *Sg = p.S + bhc * (int64_t)P * N;
        for (int e = wave; e < PT * NT; e += 4) {
            const int pt = e / NT, nt = e - pt * NT;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < ROWS / 32; ++kk) {
                const int xo = (pt * 16 + l16) * RPP + kk * 32 + 8 * g;
                const int wo = (nt * 16 + l16) * RPP + kk * 32 + 8 * g;
                if constexpr (BF) {
                    const u32x4_t xa = *(const u32x4_t *)((const uint16_t *)r1 + xo);
                    FragHL wb;
                    wb.hi = *(const u32x4_t *)((const uint16_t *)r0 + wo);
                    wb.lo = *(const u32x4_t *)((const uint16_t *)r0 + Cfg::OP_PLANE + wo);
                    acc = mma(xa, wb, acc);
                } else {
                    FragF xa, wb;
                    const f32x4_t x0 = *(const f32x4_t *)((const float *)r1 + xo);
                    const f32x4_t x1 = *(const f32x4_t *)((const float *)r1 + xo + 4);
                    const f32x4_t w0 = *(const f32x4_t *)((const float *)r0 + wo);
                    const f32x4_t w1 = *(const f32x4_t *)((const float *)r0 + wo + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        xa.v[j] = x0[j]; xa.v[j + 4] = x1[j];
                        wb.v[j] = w0[j]; wb.v[j + 4] = w1[j];
                    }
                    acc = mma(xa, wb, acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pp = pt * 16 + 4 * g + i, nn = nt * 16 + l16;
                if (pp < P && nn < N) Sg[(int64_t)pp * N + nn] = acc[i];
            }
        }
        return;
    }

    // ============================================================ output mode
    __syncthreads();  // B~ planes, X^T, angle table complete; angle table dead from here
    // H^T [p][n] from the state pass (fp32 [p][n] per chunk) into region 2
    {
        const float *Hg = p.S + (bh * p.nchunks + c) * (int64_t)P * N;
        for (int e = tid; e < PP * NP; e += 256) {
            const int pc = e / NP, n = e - pc * NP;
            const float v = (pc < P && n < N) ? Hg[(int64_t)pc * N + n] : 0.f;
            if constexpr (BF) {
                uint32_t hi, lo;
                split_hl(v, hi, lo);
                ((uint16_t *)r2)[pc * OPP + n] = (uint16_t)hi;
                ((uint16_t *)r2)[Cfg::H_PLANE + pc * OPP + n] = (uint16_t)lo;
            } else {
                ((float *)r2)[pc * OPP + n] = v;
            }
        }
    }
    __syncthreads();

    f32x4_t yin[RTW][PT], yout[RTW][PT];
#pragma unroll
    for (int k = 0; k < RTW; ++k) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            yin[k][pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            yout[k][pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        const int tt = owned_tile<NRT>(wave, k);
        if (tt >= NRT) continue;
        const int trow = tt * 16 + l16;   // this lane's t-row in the G^T fragments
        const int ttok = trow / R;
        const float cs_t = s_cs[ttok], g_t = s_gam[ttok];
        // last s-tile this t-tile reads: the one holding the last row of the tile's last token
        // (with R not dividing 16 a token's rows can continue into the next tile)
        int smax = (((tt * 16 + 15) / R) * R + R - 1) / 16;
        if (smax > NRT - 1) smax = NRT - 1;
        for (int sp = 0; sp <= smax / 2; ++sp) {
            const int st0 = 2 * sp, st1 = 2 * sp + 1;
            const bool has1 = st1 <= smax;
            // G^T tiles (s-tile, t-tile): A = B~[s rows] from LDS, B = C~[t rows] in registers
            f32x4_t g0 = {0.f, 0.f, 0.f, 0.f}, g1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const int o0 = (st0 * 16 + l16) * OPP + kk * 32 + 8 * g;
                const int o1 = (st1 * 16 + l16) * OPP + kk * 32 + 8 * g;
                if constexpr (BF) {
                    const uint16_t *hi = (const uint16_t *)r0;
                    FragHL a0;
                    a0.hi = *(const u32x4_t *)(hi + o0);
                    a0.lo = *(const u32x4_t *)(hi + Cfg::OP_PLANE + o0);
                    g0 = mma(a0, ct[k][kk], g0);
                    if (has1) {
                        FragHL a1;
                        a1.hi = *(const u32x4_t *)(hi + o1);
                        a1.lo = *(const u32x4_t *)(hi + Cfg::OP_PLANE + o1);
                        g1 = mma(a1, ct[k][kk], g1);
                    }
                } else {
                    const float *fp = (const float *)r0;
                    FragF a0;
                    const f32x4_t u0 = *(const f32x4_t *)(fp + o0), u1 = *(const f32x4_t *)(fp + o0 + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) { a0.v[j] = u0[j]; a0.v[j + 4] = u1[j]; }
                    g0 = mma(a0, ct[k][kk], g0);
                    if (has1) {
                        FragF a1;
                        const f32x4_t v0 = *(const f32x4_t *)(fp + o1), v1 = *(const f32x4_t *)(fp + o1 + 4);
#pragma unroll
                        for (int j = 0; j < 4; ++j) { a1.v[j] = v0[j]; a1.v[j + 4] = v1[j]; }
                        g1 = mma(a1, ct[k][kk], g1);
                    }
                }
            }
            // mask: slot i of g0 is G[t = trow][s = st0*16 + 4g + i]
            float m[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int s = (i < 4 ? st0 : st1) * 16 + 4 * g + (i & 3);
                const float gv = (i < 4) ? g0[i & 3] : g1[i & 3];
                const int stok = s / R;
                float L = 0.f;
                if (i < 4 || has1) {
                    if (stok < ttok) L = __expf(cs_t - s_cs[stok]) * s_scale[stok];
                    else if (stok == ttok) L = g_t;
                }
                m[i] = gv * L;
            }
            // Y_intra += M X: X fragment rows {st0*16 + 4g + 0..3, st1*16 + 4g + 0..3}
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int xo0 = (pt * 16 + l16) * RPP + st0 * 16 + 4 * g;
                const int xo1 = (pt * 16 + l16) * RPP + st1 * 16 + 4 * g;
                if constexpr (BF) {
                    const u32x2_t x0 = *(const u32x2_t *)((const uint16_t *)r1 + xo0);
                    u32x2_t x1 = {0u, 0u};
                    if (has1) x1 = *(const u32x2_t *)((const uint16_t *)r1 + xo1);
                    const u32x4_t xb = {x0[0], x0[1], x1[0], x1[1]};
                    yin[k][pt] = mma(make_hl(m), xb, yin[k][pt]);
                } else {
                    FragF xb, mf = make_f(m);
                    const f32x4_t x0 = *(const f32x4_t *)((const float *)r1 + xo0);
                    f32x4_t x1 = {0.f, 0.f, 0.f, 0.f};
                    if (has1) x1 = *(const f32x4_t *)((const float *)r1 + xo1);
#pragma unroll
                    for (int j = 0; j < 4; ++j) { xb.v[j] = x0[j]; xb.v[j + 4] = x1[j]; }
                    yin[k][pt] = mma(mf, xb, yin[k][pt]);
                }
            }
        }
        // Y_inter = C~ H: A = C~ (registers), B = H^T [p][n] planes
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int ho = (pt * 16 + l16) * OPP + kk * 32 + 8 * g;
                if constexpr (BF) {
                    FragHL hf;
                    hf.hi = *(const u32x4_t *)((const uint16_t *)r2 + ho);
                    hf.lo = *(const u32x4_t *)((const uint16_t *)r2 + Cfg::H_PLANE + ho);
                    yout[k][pt] = mma(ct[k][kk], hf, yout[k][pt]);
                } else {
                    FragF hf;
                    const f32x4_t v0 = *(const f32x4_t *)((const float *)r2 + ho);
                    const f32x4_t v1 = *(const f32x4_t *)((const float *)r2 + ho + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) { hf.v[j] = v0[j]; hf.v[j + 4] = v1[j]; }
                    yout[k][pt] = mma(ct[k][kk], hf, yout[k][pt]);
                }
            }
        }
    }
    __syncthreads();  // everyone done with the B~ planes: region 0 becomes the y staging
    ET *ys = (ET *)r0;
    const float Dh = p.D[h];
#pragma unroll
    for (int k = 0; k < RTW; ++k) {
        const int tt = owned_tile<NRT>(wave, k);
        if (tt >= NRT) continue;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = tt * 16 + 4 * g + i, pc = pt * 16 + l16;
                const int tok = row / R;
                float xv;
                if constexpr (BF) xv = bf2f(((const uint16_t *)r1)[pc * RPP + row]);
                else xv = ((const float *)r1)[pc * RPP + row];
                const float v = yin[k][pt][i] + s_ecs[tok] * yout[k][pt][i] + Dh * xv;
                Io::st(ys + row * PP + pc, v);
            }
        }
    }
    __syncthreads();
    {
        ET *yg = (ET *)p.y;
        for (int e = tid; e < Rv * PP; e += 256) {
            const int row = e / PP, pc = e - row * PP;
            if (pc >= P) continue;
            const int tok = row / R, r = row - tok * R;
            yg[((b * T + t0 + tok) * H + h) * P * R + pc * R + r] = ys[row * PP + pc];
        }
    }
    if (want_final) {
        // carried x of the last token and the final angle
        const int lrow0 = (Qv - 1) * R;
        for (int e = tid; e < P * R; e += 256) {
            const int pc = e / R, r = e - pc * R;
            float xv;
            if constexpr (BF) xv = bf2f(((const uint16_t *)r1)[pc * RPP + lrow0 + r]);
            else xv = ((const float *)r1)[pc * RPP + lrow0 + r];
            p.px1[(bh * P + pc) * R + r] = xv;
        }
        for (int i = tid; i < N2; i += 256) p.ang1[bh * N2 + i] = thfin[i];
    }
}

// ---------------------------------------------------------------- dispatch
template <class Io, int ROWS, int NP, int PP, int MODE>
static hipError_t launch_one(const ScanParams &p, hipStream_t stream) {
    using Cfg = ChunkCfg<Io, ROWS, NP, PP, MODE>;
    auto kern = chunk_kernel<Io, ROWS, NP, PP, MODE>;
    if (Cfg::BYTES > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)Cfg::BYTES);
        if (e != hipSuccess) return e;
    }
    dim3 grid((unsigned)p.nchunks, (unsigned)p.H, (unsigned)p.B);
    hipLaunchKernelGGL(kern, grid, dim3(256), Cfg::BYTES, stream, p);
    return hipGetLastError();
}

template <class Io, int MODE>
static size_t bytes_of(const TileShape &ts) {
#define M3_CASE(RW, NPV, PPV) \
    if (ts.rows == RW && ts.np == NPV && ts.pp == PPV) return ChunkCfg<Io, RW, NPV, PPV, MODE>::BYTES;
#define M3_PP(RW, NPV) M3_CASE(RW, NPV, 32) M3_CASE(RW, NPV, 64) M3_CASE(RW, NPV, 128)
#define M3_NP(RW) M3_PP(RW, 32) M3_PP(RW, 64) M3_PP(RW, 128)
    M3_NP(32) M3_NP(64) M3_NP(128)
#undef M3_CASE
    return 0;
}

template <class Io, int MODE>
static hipError_t launch_mode(const TileShape &ts, const ScanParams &p, hipStream_t stream) {
#define M3_CASE(RW, NPV, PPV) \
    if (ts.rows == RW && ts.np == NPV && ts.pp == PPV) return launch_one<Io, RW, NPV, PPV, MODE>(p, stream);
    M3_NP(32) M3_NP(64) M3_NP(128)
#undef M3_CASE
#undef M3_PP
#undef M3_NP
    return hipErrorInvalidValue;
}

size_t chunk_kernel_lds_bytes(int mode, bool bf16, const TileShape &ts) {
    if (bf16) return mode == MODE_STATE ? bytes_of<IoBF16, MODE_STATE>(ts) : bytes_of<IoBF16, MODE_OUTPUT>(ts);
    return mode == MODE_STATE ? bytes_of<IoF32, MODE_STATE>(ts) : bytes_of<IoF32, MODE_OUTPUT>(ts);
}

hipError_t launch_chunk_kernel(int mode, bool bf16, const TileShape &ts, const ScanParams &p,
                               hipStream_t stream) {
    if (bf16) {
        return mode == MODE_STATE ? launch_mode<IoBF16, MODE_STATE>(ts, p, stream)
                                  : launch_mode<IoBF16, MODE_OUTPUT>(ts, p, stream);
    }
    return mode == MODE_STATE ? launch_mode<IoF32, MODE_STATE>(ts, p, stream)
                              : launch_mode<IoF32, MODE_OUTPUT>(ts, p, stream);
}

}  // namespace m3
