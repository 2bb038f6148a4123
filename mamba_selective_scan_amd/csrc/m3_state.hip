// m3_state.hip -- the empty-call state copy and the single-token decode step.
#include <type_traits>

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

// ---------------------------------------------------------------- empty call
// T == 0: the final state is the initial state (zeros when there is none);
// the angle is reduced to [0, 2 pi).
__global__ __launch_bounds__(256) void fill_state_kernel(ScanParams p) {
    const int64_t nbh = p.B * p.H;
    const int64_t nh = nbh * p.N * p.P, nb = nbh * p.N * p.R, nx = nbh * p.P * p.R, na = nbh * p.nr;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool have = p.h0 && p.pB0 && p.px0 && (p.ang0 || p.nr == 0);
    if (gid < nh) p.h1[gid] = have ? p.h0[gid] : 0.f;
    if (gid < nb) p.pB1[gid] = have ? p.pB0[gid] : 0.f;
    if (gid < nx) p.px1[gid] = have ? p.px0[gid] : 0.f;
    if (gid < na) p.ang1[gid] = have ? (float)wrap_2pi((double)p.ang0[gid]) : 0.f;
}

hipError_t launch_fill_state(const ScanParams &p, hipStream_t stream) {
    const int64_t nbh = p.B * p.H;
    int64_t m = nbh * p.N * p.P;
    if (nbh * p.N * p.R > m) m = nbh * p.N * p.R;
    if (nbh * p.P * p.R > m) m = nbh * p.P * p.R;
    if (m == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_state_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------- decode step
// alpha, beta, gamma of the step's token: dt and lambda through the optional input
// activations, A per head or (one token) per (batch, head).
__device__ __forceinline__ void step_coeffs(const StepParams &p, int64_t b, int h, float &alpha, float &beta,
                                            float &gamma) {
    float dt = p.dt[b * p.rsdt + h], lam = p.lam[b * p.rslam + h];
    if (p.flags & kFlagDtSoftplus) dt = softplus_f(dt + (p.dtbias ? p.dtbias[h] : 0.f));
    if (p.flags & kFlagLamSigmoid) lam = sigmoid_f(lam);
    const float A = (p.flags & kFlagAPerToken) ? p.A[b * p.rsa + h] : p.A[h];
    alpha = __expf(dt * A);
    beta = alpha * dt * (1.f - lam);
    gamma = lam * dt;
}

// A value rounded to the io type (bf16 inputs formed in fp32, such as x expanded by mimo_x,
// are rounded once, as the scan rounds them).
template <class Io>
__device__ __forceinline__ float round_io(float v) {
    if constexpr (Io::bytes == 2) return bf2f(f2bf(v));
    else return v;
}
// Load of base[off] when ok, else of base[0] (base must be a valid array): the value is
// selected afterwards, so that a run of such loads is in flight before the first use.
template <class T>
__device__ __forceinline__ T ld_sel(const T *base, int64_t off, bool ok) { return base[ok ? off : 0]; }
template <class Io>
__device__ __forceinline__ float to_f(typename Io::T v) {
    if constexpr (Io::bytes == 2) return bf2f(v);
    else return v;
}

// One workgroup per (head, batch).  The step is the recurrence itself for one
// token (torchmamba "Quickstart": step(u_t, cache)):
//     Theta <- Theta + theta;  B~, C~ = Rot(Theta)(norm(B) + bias), ...
//     h <- alpha h + beta sum_r prevB_r prevx_r^T + gamma sum_r B~_r x_r^T
//     y_r = h^T C~_r + D x_r;  prev_B <- B~;  prev_x <- x
// Memory-bound: h is read once and written once with 16-byte accesses; the
// first U rows of h per thread are requested before the prologue so that their
// latency overlaps the norm and rotation.
template <class Io, int VEC, int RMAX>
__global__ __launch_bounds__(256) void step_kernel(StepParams p) {
    using ET = typename Io::T;
    constexpr int U = 4;  // h rows in flight per thread
    const int h = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int N = p.N, P = p.P, R = RMAX == 1 ? 1 : p.R, N2 = N / 2;
    const int64_t bh = b * p.H + h;  // == (b, t=0, h) since T = 1
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    M3_DCHECK(p, b < p.B && h < p.H && R <= RMAX && P % VEC == 0 && 256 / (P / VEC) >= 1);

    // state update mapping: thread = (group of VEC columns, n group)
    const int PG = P / VEC;
    const int NG = 256 / PG;
    const int pg = tid % PG, ng = tid / PG;
    const bool upd = ng < NG;
    float *hst = p.h + bh * (int64_t)N * P;
    float hv[U][VEC];
    auto load_rows = [&](int n0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int n = n0 + u * NG;
            if (upd && n < N) {
                if constexpr (VEC == 4) {
                    const f32x4_t v4 = *(const f32x4_t *)(hst + (int64_t)n * P + pg * 4);
#pragma unroll
                    for (int j = 0; j < VEC; ++j) hv[u][j] = v4[j];
                } else {
                    hv[u][0] = hst[(int64_t)n * P + pg];
                }
            }
        }
    };
    load_rows(ng);

    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *s_bt = sm;              // [N][R] new B~ (raw B first)
    float *s_ct = s_bt + N * R;    // [N][R] new C~ (raw C first)
    float *s_pb = s_ct + N * R;    // [N][R] previous B~
    float *s_px = s_pb + N * R;    // [P][R] previous x
    float *s_x = s_px + P * R;     // [P][R] x
    float *s_cos = s_x + P * R;    // [N/2]
    float *s_sin = s_cos + N2;     // [N/2]
    float *s_rs = s_sin + N2;      // [2][R] norm factors (B then C)
    float *s_red = s_rs + 2 * R;   // [NG][P][R] partial outputs

    // the token's rows (row b of each input; strided slices allowed), at head h
    const ET *xg = (const ET *)p.x + b * p.rsx + (int64_t)h * P * (p.mx ? 1 : R);
    const ET *bg = (const ET *)p.Bm + b * p.rsb + (int64_t)h * N * R;
    const ET *cg = (const ET *)p.Cm + b * p.rsc + (int64_t)h * N * R;
    for (int e = tid; e < N * R; e += 256) {
        s_bt[e] = Io::ld(bg + e);
        s_ct[e] = Io::ld(cg + e);
        s_pb[e] = p.pB[bh * N * R + e];
    }
    for (int e = tid; e < P * R; e += 256) {
        if (p.mx) {  // rank-free x expanded by the learned vector of rank r
            const int pc = e / R, r = e - pc * R;
            s_x[e] = round_io<Io>(Io::ld(xg + pc) * p.mx[((int64_t)h * R + r) * P + pc]);
        } else {
            s_x[e] = Io::ld(xg + e);
        }
        s_px[e] = p.px[bh * P * R + e];
    }
    for (int i = tid; i < N2; i += 256) {
        float sn = 0.f, cn = 1.f;  // pairs past nr do not rotate
        if (i < p.nr) {
            const double th =
                wrap_2pi((double)p.ang[bh * p.nr + i] + (double)p.theta[b * p.rsth + (int64_t)h * p.nr + i]);
            sincosf((float)th, &sn, &cn);
            p.ang[bh * p.nr + i] = (float)th;
        }
        s_cos[i] = cn;
        s_sin[i] = sn;
    }
    __syncthreads();
    // RMS over N per (B or C, rank): one wave per combination
    const bool bcnorm = (p.flags & kFlagNorm) != 0;
    for (int cb = wave; cb < 2 * R; cb += 4) {
        const float *src = cb < R ? s_bt : s_ct;
        const int r = cb < R ? cb : cb - R;
        float ss = 0.f;
        for (int n = lane; n < N; n += 64) ss += src[n * R + r] * src[n * R + r];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
        if (lane == 0) s_rs[cb] = bcnorm ? rsqrtf(ss / (float)N + p.eps) : 1.f;
    }
    __syncthreads();
    // norm, gain, bias, rotation: one thread per (pair, rank); the pair's components are
    // adjacent, or one in each half of N (half-split pairing)
    const bool hsplit = (p.flags & kFlagHalfSplit) != 0;
    for (int e = tid; e < N2 * R; e += 256) {
        const int i = e / R, r = e - i * R;
        const int n0 = hsplit ? i : 2 * i, n1 = hsplit ? i + N2 : 2 * i + 1;
        const float rb = s_rs[r], rc = s_rs[R + r];
        float gb0 = 1.f, gb1 = 1.f, gc0 = 1.f, gc1 = 1.f;
        if (bcnorm && p.bnw) { gb0 = p.bnw[n0]; gb1 = p.bnw[n1]; }
        if (bcnorm && p.cnw) { gc0 = p.cnw[n0]; gc1 = p.cnw[n1]; }
        float u = s_bt[n0 * R + r] * rb * gb0, w = s_bt[n1 * R + r] * rb * gb1;
        float uc = s_ct[n0 * R + r] * rc * gc0, wc = s_ct[n1 * R + r] * rc * gc1;
        if (p.bbias) {
            u += p.bbias[((int64_t)h * R + r) * N + n0];
            w += p.bbias[((int64_t)h * R + r) * N + n1];
        }
        if (p.cbias) {
            uc += p.cbias[((int64_t)h * R + r) * N + n0];
            wc += p.cbias[((int64_t)h * R + r) * N + n1];
        }
        const float cn = s_cos[i], sn = s_sin[i];
        s_bt[n0 * R + r] = u * cn - w * sn;
        s_bt[n1 * R + r] = u * sn + w * cn;
        s_ct[n0 * R + r] = uc * cn - wc * sn;
        s_ct[n1 * R + r] = uc * sn + wc * cn;
    }
    __syncthreads();
    for (int e = tid; e < N * R; e += 256) p.pB[bh * N * R + e] = s_bt[e];
    for (int e = tid; e < P * R; e += 256) p.px[bh * P * R + e] = s_x[e];

    float alpha, beta, gamma;
    step_coeffs(p, b, h, alpha, beta, gamma);

    float acc[VEC][RMAX];
#pragma unroll
    for (int j = 0; j < VEC; ++j)
#pragma unroll
        for (int r = 0; r < RMAX; ++r) acc[j][r] = 0.f;
    if (upd) {
        for (int n0 = ng; n0 < N; n0 += U * NG) {
            if (n0 != ng) load_rows(n0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int n = n0 + u * NG;
                if (n >= N) break;
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const int pc = pg * VEC + j;
                    float prev = 0.f, cur = 0.f;
                    for (int r = 0; r < R; ++r) {
                        prev += s_pb[n * R + r] * s_px[pc * R + r];
                        cur += s_bt[n * R + r] * s_x[pc * R + r];
                    }
                    const float hn = alpha * hv[u][j] + beta * prev + gamma * cur;
                    hv[u][j] = hn;
#pragma unroll
                    for (int r = 0; r < RMAX; ++r)
                        if (r < R) acc[j][r] += hn * s_ct[n * R + r];
                }
                if constexpr (VEC == 4) {
                    *(f32x4_t *)(hst + (int64_t)n * P + pg * 4) = f32x4_t{hv[u][0], hv[u][VEC > 1 ? 1 : 0],
                                                                          hv[u][VEC > 2 ? 2 : 0], hv[u][VEC > 3 ? 3 : 0]};
                } else {
                    hst[(int64_t)n * P + pg] = hv[u][0];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j)
#pragma unroll
            for (int r = 0; r < RMAX; ++r)
                if (r < R) s_red[(ng * P + pg * VEC + j) * R + r] = acc[j][r];
    }
    __syncthreads();
    const float Dh = p.D[h];
    const ET *zg = p.z ? (const ET *)p.z + b * p.rsz + (int64_t)h * P * (p.mz ? 1 : R) : nullptr;
    ET *yg = (ET *)p.y + b * p.rsy + (int64_t)h * P * (p.mo ? 1 : R);
    // output (pc, r) with the optional gate y * silu(z_r)
    auto y_of = [&](int pc, int r) {
        const int e = pc * R + r;
        float s = 0.f;
        for (int k = 0; k < NG; ++k) s += s_red[k * P * R + e];
        float v = s + Dh * s_x[e];
        if (zg) {
            const float zv = p.mz ? Io::ld(zg + pc) * p.mz[((int64_t)h * R + r) * P + pc] : Io::ld(zg + e);
            v *= silu_f(zv);
        }
        return v;
    };
    if (p.mo) {  // rank contraction y[pc] = sum_r mimo_o[h, r, pc] y_r[pc]
        for (int pc = tid; pc < P; pc += 256) {
            float acc_o = 0.f;
            for (int r = 0; r < R; ++r) acc_o += p.mo[((int64_t)h * R + r) * P + pc] * y_of(pc, r);
            Io::st(yg + pc, acc_o);
        }
    } else {
        for (int e = tid; e < P * R; e += 256) Io::st(yg + e, y_of(e / R, e % R));
    }
    (void)lane;
}

// Rank-1 decode step (P a multiple of 4).  B~ and C~ are formed by one wave each (lane n
// holds component n, and n + 64 when N > 64): a wave reduction for the norm and a swap
// between neighbouring lanes for the rotation of pair (2i, 2i + 1).  A third wave stages
// x and the carried x, a fourth computes the step's coefficients.  The step then needs two
// workgroup barriers, each thread's rows of h are requested before anything else, and each
// wave issues all of its loads before the first use.  The state rows are read and written
// with the non-temporal hint (each is touched once per step; measured about 2% faster).
template <class Io>
__global__ __launch_bounds__(256) void step_kernel_r1(StepParams p) {
    using ET = typename Io::T;
    constexpr int U = 4;  // h rows in flight per thread
    const int h = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int N = p.N, P = p.P, N2 = N / 2;
    const int64_t bh = b * p.H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    M3_DCHECK(p, b < p.B && h < p.H && p.R == 1 && P % 4 == 0 && N <= 128);
    const int PG = P / 4, NG = 256 / PG;
    const int pg = tid % PG, ng = tid / PG;
    const bool upd = ng < NG;
    float *hst = p.h + bh * (int64_t)N * P;
    f32x4_t hv[U];
    auto load_rows = [&](int n0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int n = n0 + u * NG;
            if (upd && n < N) hv[u] = __builtin_nontemporal_load((const f32x4_t *)(hst + (int64_t)n * P + pg * 4));
        }
    };
    load_rows(ng);

    extern __shared__ __attribute__((aligned(16))) float sm[];
    const int NA = (N + 3) & ~3, PA = (P + 3) & ~3, N2A = (N2 + 3) & ~3;  // 16-byte aligned parts
    float *s_bt = sm;             // [N] B~
    float *s_ct = s_bt + NA;      // [N] C~
    float *s_pb = s_ct + NA;      // [N] previous B~
    float *s_x = s_pb + NA;       // [P] x
    float *s_px = s_x + PA;       // [P] previous x
    float *s_ang = s_px + PA;     // [N/2] new angle
    float *s_cf = s_ang + N2A;    // [4] alpha, beta, gamma
    float *s_red = s_cf + 4;      // [NG][P] partial outputs
    const bool bcnorm = (p.flags & kFlagNorm) != 0;
    // Every load of a wave is issued before its first use (absent elements load offset 0 of a
    // valid array and are replaced afterwards): wave 0 stages B~ (and swaps prev_B), wave 1
    // C~, wave 2 x (and swaps prev_x), wave 3 the step's coefficients.
    if (wave < 2) {
        const ET *src = wave == 0 ? (const ET *)p.Bm + b * p.rsb + (int64_t)h * N : (const ET *)p.Cm + b * p.rsc + (int64_t)h * N;
        const float *gain = wave == 0 ? p.bnw : p.cnw;
        const float *bias = wave == 0 ? p.bbias : p.cbias;
        const bool hg = bcnorm && gain != nullptr, hb = bias != nullptr;
        const float *gp = hg ? gain : p.dt, *bp = hb ? bias + (int64_t)h * N : p.dt;
        // angle and increment of this (batch, head), rebased so that pair i is at offset i
        const bool rot = p.nr > 0 && p.ang && p.theta;
        const float *ap = rot ? p.ang + bh * p.nr : p.dt, *tp = rot ? p.theta + b * p.rsth + (int64_t)h * p.nr : p.dt;
        ET raw[2];
        float gv[2], bv[2], av[2], tv[2], pbv[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int n = lane + 64 * k, i = n >> 1;
            const bool in = n < N, ir = in && i < p.nr;
            raw[k] = ld_sel(src, n, in);
            gv[k] = ld_sel(gp, n, in && hg);
            bv[k] = ld_sel(bp, n, in && hb);
            av[k] = ld_sel(ap, i, ir);
            tv[k] = ld_sel(tp, i, ir);
            pbv[k] = ld_sel(p.pB, bh * N + n, in && wave == 0);
        }
        float v[2], ss = 0.f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            v[k] = lane + 64 * k < N ? to_f<Io>(raw[k]) : 0.f;
            ss += v[k] * v[k];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
        const float rs = bcnorm ? rsqrtf(ss / (float)N + p.eps) : 1.f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int n = lane + 64 * k;
            const bool in = n < N;
            float u = v[k] * rs;
            if (in && hg) u *= gv[k];
            if (in && hb) u += bv[k];
            // the pair's angle Theta + theta (the stored angle is kept in [0, 2 pi))
            const int i = n >> 1;
            const double a = (in && i < p.nr) ? wrap_2pi((double)av[k] + (double)tv[k]) : 0.0;
            const f32x2_t sc = sincos_acc((float)a);  // (sin, cos)
            const float other = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(u), 0xB1, 0xF, 0xF, false));
            const float out = (n & 1) ? other * sc[0] + u * sc[1] : u * sc[1] - other * sc[0];
            if (!in) continue;
            if (wave == 0) {
                s_pb[n] = pbv[k];
                p.pB[bh * N + n] = out;
                s_bt[n] = out;
                if ((n & 1) == 0) s_ang[i] = (float)a;
            } else {
                s_ct[n] = out;
            }
        }
    } else if (wave == 2) {
        const ET *xg = (const ET *)p.x + b * p.rsx + (int64_t)h * P;
        for (int pc = lane; pc < P; pc += 64) {
            const float xv = Io::ld(xg + pc), pxv = p.px[bh * P + pc];
            s_x[pc] = xv;
            s_px[pc] = pxv;
            p.px[bh * P + pc] = xv;
        }
    } else if (lane == 0) {
        float alpha, beta, gamma;
        step_coeffs(p, b, h, alpha, beta, gamma);
        s_cf[0] = alpha;
        s_cf[1] = beta;
        s_cf[2] = gamma;
    }
    // the gate input of this thread's first output element
    const ET *zb = p.z ? (const ET *)p.z + b * p.rsz + (int64_t)h * P : (const ET *)p.x;
    const ET zr = ld_sel(zb, tid, p.z != nullptr && tid < P);
    __syncthreads();
    if (tid < p.nr) p.ang[bh * p.nr + tid] = s_ang[tid];

    const float alpha = s_cf[0], beta = s_cf[1], gamma = s_cf[2];
    if (upd) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        f32x4_t xv4 = *(const f32x4_t *)(s_x + pg * 4), pxv4 = *(const f32x4_t *)(s_px + pg * 4);
        for (int n0 = ng; n0 < N; n0 += U * NG) {
            if (n0 != ng) load_rows(n0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int n = n0 + u * NG;
                if (n >= N) break;
                const float pb = beta * s_pb[n], bt = gamma * s_bt[n], ct = s_ct[n];
                f32x4_t hn;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    hn[j] = alpha * hv[u][j] + pb * pxv4[j] + bt * xv4[j];
                    acc[j] += hn[j] * ct;
                }
                __builtin_nontemporal_store(hn, (f32x4_t *)(hst + (int64_t)n * P + pg * 4));
            }
        }
        *(f32x4_t *)(s_red + ng * P + pg * 4) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    }
    __syncthreads();
    const float Dh = p.D[h];
    for (int e = tid; e < P; e += 256) {
        float sacc = 0.f;
        for (int k2 = 0; k2 < NG; ++k2) sacc += s_red[k2 * P + e];
        float v = sacc + Dh * s_x[e];
        if (p.z) v *= silu_f(e == tid ? to_f<Io>(zr) : Io::ld(zb + e));
        Io::st((ET *)p.y + b * p.rsy + (int64_t)h * P + e, v);
    }
}

static size_t step_lds_bytes(const StepParams &p, int vec) {
    const int NG = 256 / (p.P / vec);
    return sizeof(float) * (size_t)(3 * p.N * p.R + 2 * p.P * p.R + p.N + 2 * p.R + NG * p.P * p.R);
}

hipError_t launch_step(bool bf16, const StepParams &p, hipStream_t stream) {
    // rank 1 with adjacent pairs (swapped between neighbouring lanes) and no MIMO projection
    if (p.R == 1 && p.P % 4 == 0 && !(p.flags & kFlagHalfSplit) && !p.mx && !p.mz && !p.mo) {
        const int NG = 256 / (p.P / 4);
        const int NA = (p.N + 3) & ~3, PA = (p.P + 3) & ~3, N2A = (p.N / 2 + 3) & ~3;
        const size_t lds = sizeof(float) * (size_t)(3 * NA + 2 * PA + N2A + 4 + NG * p.P);
        dim3 grid((unsigned)p.H, (unsigned)p.B);
        if (bf16) hipLaunchKernelGGL((step_kernel_r1<IoBF16>), grid, dim3(256), lds, stream, p);
        else hipLaunchKernelGGL((step_kernel_r1<IoF32>), grid, dim3(256), lds, stream, p);
        return hipGetLastError();
    }
    const int vec = (p.P % 4 == 0) ? 4 : 1;
    const size_t lds = step_lds_bytes(p, vec);
    dim3 grid((unsigned)p.H, (unsigned)p.B);
#define M3_STEP_LAUNCH(IO, V, RM) hipLaunchKernelGGL((step_kernel<IO, V, RM>), grid, dim3(256), lds, stream, p)
    if (bf16) {
        if (p.R == 1) { if (vec == 4) M3_STEP_LAUNCH(IoBF16, 4, 1); else M3_STEP_LAUNCH(IoBF16, 1, 1); }
        else { if (vec == 4) M3_STEP_LAUNCH(IoBF16, 4, 8); else M3_STEP_LAUNCH(IoBF16, 1, 8); }
    } else {
        if (p.R == 1) { if (vec == 4) M3_STEP_LAUNCH(IoF32, 4, 1); else M3_STEP_LAUNCH(IoF32, 1, 1); }
        else { if (vec == 4) M3_STEP_LAUNCH(IoF32, 4, 8); else M3_STEP_LAUNCH(IoF32, 1, 8); }
    }
#undef M3_STEP_LAUNCH
    return hipGetLastError();
}

}  // namespace m3
