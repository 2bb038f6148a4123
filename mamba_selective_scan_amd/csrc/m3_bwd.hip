// m3_bwd.hip -- gradients of the chunked Mamba-3 scan (reverse mode) on gfx950.
//
// The pages ask for the scan to be differentiable (torchmamba "Verification":
// fp64 gradchecks of the scans; dotLLM PR #136: the block trains) and print no
// backward algorithm.  This is the adjoint of the chunked forward: the same
// single-scan form of the trapezoid (dotLLM PR #136, "Mamba-3 streaming decode":
// shifted state g_t = h_t + eta_t B~_t x_t^T with eta_t = dt_{t+1}(1 - lambda_{t+1}))
// and the same chunk decomposition (torchmamba README, "Math notes", M2 chunked
// SSD; M3 RoPE trick: B and C rotated by the cumulative angle, so the state
// carries no rotation inside a chunk).  Per chunk of 64 rows ((token, rank)
// pairs), in the chunk's own rotation frame (angles summed from the chunk start):
//     Y   = (L o C~ B~^T) X + diag(e^cs) C~ H,          H: state before the chunk
//     H'  = Rot(-Phi_end) (e^cs_end H + S),   S = sum_s e^(cs_end - cs_s) kappa_s B~_s x_s^T
//     L[t, s] = e^(cs_t - cs_s) kappa_s (token(t) > token(s)), gamma_t (same token), 0 (earlier)
// with kappa = gamma + eta.  With Gb the adjoint of the state after the chunk:
//     dX   = (L o G)^T dY + diag(e^(cs_end - cs) kappa) B~ Gb + D dY,      G = C~ B~^T
//     dC~  = (L o dY X^T) B~ + diag(e^cs) dY H^T
//     dB~  = (L o dY X^T)^T C~ + diag(e^(cs_end - cs) kappa) X Gb^T
//     d cs_t: row sums minus column sums of L o G o dY X^T over strictly earlier tokens,
//             plus C~_t . (state term of dC~_t), minus kappa_s B~_s . (state term of dB~_s / kappa_s);
//             at the chunk's last token also e^cs_end <Gb, H> + the sum of the latter
//     d log alpha_k = sum of d cs over the chunk's tokens t >= k
//     d Theta_t (per pair) = <dC~_t, J C~_t> + <dB~_t, J B~_t>,   J = [[0, -1], [1, 0]]
//     d theta_k = sum of d Theta over all tokens t >= k (+ the final angle's gradient)
// The state adjoints obey
//     Gb(before chunk) = Rot(Phi_end of the previous chunk) (e^cs_end Gb + sum_t e^cs_t C~_t dy_t^T).
// Kernels, in launch order:
//   bwd_chunk_state_kernel  per chunk: S and U = sum_t e^cs_t C~_t dy_t^T (MFMA), chunk totals
//   bwd_state_pass_kernel   per (sequence, pair, column): states before each chunk (forward
//                           over the chunks) and adjoints after each chunk (reverse), in place
//   bwd_chunk_grad_kernel   per chunk: every gradient above (ten MFMA products), the norm
//                           backward, local angle sums, per-token scalar gradients
//   bwd_angle_suffix_kernel per sequence: angle gradient sums of the later chunks
//   bwd_init_kernel         per sequence: gradients of the initial state (angle: frame rotation)
//   bwd_token_kernel        per chunk: dt, lambda, A gradients; angle gradients completed
//   bwd_reduce_kernel       parameter gradients (fixed-order sums of per-chunk records)
//
// Matrix cores: v_mfma_f32_16x16x4_f32 on fp32 operands (full fp32 products for
// every I/O type).  A 32-wide contraction chunk is a fragment of 8 values per lane,
// slot j of lane group g carrying logical index 8 g + j (or, for operands taken
// from result tiles, 16 a + 4 g + j over a pair of tiles); A and B agree on it.
// Eight waves per chunk: wave (w, half) owns rows 16 w .. 16 w + 15 of the chunk and
// half of the output column tiles.
#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

namespace {

constexpr int kRows = 64;     // rows per chunk
constexpr int kWaves = 8;     // waves per chunk workgroup
constexpr int kThreads = 64 * kWaves;

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
// sum over the wave, returned to every lane: row sums, then rows 0+1 and 2+3 (row_bcast:15
// into rows 1 and 3), then all four (row_bcast:31 into rows 2 and 3); lane 63 holds the total
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum16(v);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// sum over each half of the wave (lanes 0..31, 32..63), returned to every lane of that half:
// row sums, then rows 0+1 and 2+3 (row_bcast:15 into rows 1 and 3); lanes 31 and 63 hold them
__device__ __forceinline__ float half_sum(float v) {
    v = row_sum16(v);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    return (threadIdx.x & 32) ? hi : lo;
}
// Row passes over the B and C rows: with at most 32 pairs a wave takes two rows per
// instruction (lanes 0..31 and 32..63, lane = pair), otherwise one (lane = pair).
template <int N2P>
struct RowPass {
    static constexpr bool HV = N2P <= 32;
    static constexpr int NM = HV ? 4 : 8;  // rows per wave: wv + 8 (NM-step index)
    __device__ static int half() { return HV ? (int)((threadIdx.x >> 5) & 1) : 0; }
    __device__ static int pair() { return HV ? (int)(threadIdx.x & 31) : (int)(threadIdx.x & 63); }
    __device__ static int row(int wv, int m) { return wv + 8 * (HV ? 2 * m + half() : m); }
    __device__ static float sum(float v) { return HV ? half_sum(v) : wave_sum(v); }
    // the other half's value of v (0 when a row of the wave takes every lane)
    __device__ static float other(float v) {
        if constexpr (HV) {
            // permlane32_swap of v with itself: [0] holds lane l & 31's value, [1] lane (l & 31) + 32's
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
        } else {
            return 0.f;
        }
    }
};

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
// Branch-free loads: an absent element is loaded from offset 0 and replaced by 0 afterwards,
// so that a run of loads is issued before the first wait (a load inside a divergent branch
// whose value is used in that branch costs a full memory round trip each).
template <class T>
__device__ __forceinline__ T ld_raw(const T *base, int64_t off, bool ok) { return base[ok ? off : 0]; }
template <class Io>
__device__ __forceinline__ float raw_f(typename Io::T v, bool ok) {
    float f;
    if constexpr (Io::bytes == 2) f = bf2f(v);
    else f = v;
    return ok ? f : 0.f;
}
// acc += A B over one 32-wide contraction chunk (slot j -> instruction j)
__device__ __forceinline__ f32x4_t mma8(const float (&a)[8], const float (&b)[8], f32x4_t acc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = mfma_f(a[j], b[j], acc);
    return acc;
}
// logical contraction index of slot j for operands taken from result tiles 2 kc and 2 kc + 1
__device__ __forceinline__ int tile_k(int kc, int g, int j) { return 32 * kc + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4); }

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
// eta_t = dt_{t+1} (1 - lambda_{t+1}), 0 at the last token (t = -1 gives the initial state's)
__device__ __forceinline__ float eta_at(const BwdParams &p, int64_t b, int h, int64_t t) {
    if (t + 1 >= p.T) return 0.f;
    float dt, lam, u, v;
    act_scalars(p, (b * p.T + t + 1) * p.H + h, h, dt, lam, u, v);
    return dt * (1.f - lam);
}

// LDS layout of the chunk kernels (floats).  GRAD: the gradient kernel's layout, which keeps
// the chunk's running angles (PH) and the rows' norm factors (RS) for the norm backward when
// they fit beside the rest; otherwise the angles share the slab area and are computed again.
// SPLIT (chunk-state kernel): one B~/C~ tile and one x/dy tile, staged one side at a time.
// Columns of rotation pair i (i < NPAD / 2): (2i, 2i + 1); with the half-split pairing
// (i, i + N/2) for i < N/2, and the padding columns N + 2(i - N/2) and the next beyond, so that
// every lane of a pair-per-lane pass owns two columns of its own.
__device__ __forceinline__ int pn0(const BwdParams &p, int i) {
    const int h = p.N >> 1;
    return !p.hs ? 2 * i : (i < h ? i : p.N + 2 * (i - h));
}
__device__ __forceinline__ int pn1(const BwdParams &p, int i) {
    const int h = p.N >> 1;
    return !p.hs ? 2 * i + 1 : (i < h ? i + h : p.N + 2 * (i - h) + 1);
}

// The same map in the chunk kernels, where the half-split pairing (HS) needs N = NPAD: pair i
// is (2i, 2i + 1), or (i, i + NPAD/2), at compile time.
template <bool HS, int NPAD>
__device__ __forceinline__ constexpr int pc0(int i) { return HS ? i : 2 * i; }
template <bool HS, int NPAD>
__device__ __forceinline__ constexpr int pc1(int i) { return HS ? i + NPAD / 2 : 2 * i + 1; }

template <int NPAD, int PPAD, bool GRAD = false, bool SPLIT = false>
struct CL {
    static constexpr int BP = NPAD + 1, XP = PPAD + 1, N2P = NPAD / 2;
    static constexpr int SB = 0;                                  // [64][BP] B~ rows (then dB~)
    static constexpr int SC = SPLIT ? SB : SB + kRows * BP;       // [64][BP] C~ rows (then dC~)
    static constexpr int SX = SC + kRows * BP;                    // [64][XP] x rows
    static constexpr int SY = SPLIT ? SX : SX + kRows * XP;       // [64][XP] gated dy rows
    static constexpr int SS = SY + kRows * XP;                    // state slab [32][XP]
    static constexpr int REST = 3 * 64 + 6 * 64 + 8 * 64 + 64 + 128 + 128 + 32;
    static constexpr bool KEEP = GRAD && (SS + 32 * XP + kRows * N2P + 128 + REST) * 4 <= 160 * 1024;
    static constexpr int SLAB = !GRAD ? kRows * N2P : KEEP ? 32 * XP : (32 * XP > kRows * N2P ? 32 * XP : kRows * N2P);
    static constexpr int PH = KEEP ? SS + SLAB : SS;  // [64][N2P] running angles of the chunk
    static constexpr int RS = PH + kRows * N2P;     // [2][64] norm factors of the B and C rows (KEEP)
    static constexpr int TK = KEEP ? RS + 128 : SS + SLAB;  // per token: cs, kappa, gamma
    static constexpr int RT = TK + 3 * 64;          // per row: cs, kappa, gamma, token, e^(cs_end-cs), e^cs
    static constexpr int RW = RT + 6 * 64;          // [4][64] strict row sums (with RD: [8][64] scan scratch)
    static constexpr int RD = RW + 4 * 64;          // [4][64] same-token row sums
    static constexpr int CE = RD + 4 * 64;          // [64] strict column sums
    static constexpr int AT = CE + 64;              // [2][64] C~ . (state term of dC~) per row
    static constexpr int KS = AT + 128;             // [2][64] B~ . (state term of dB~ / kappa) per row
    static constexpr int MS = KS + 128;             // misc
    // [8 waves][4 tiles][64 lanes][4] exchange of the s-oriented triangle's G and dY X^T tiles
    // between the two waves of a row tile (gradient kernel, when it fits)
    static constexpr int XC = MS + 32;
    static constexpr bool XCH = GRAD && (XC + kWaves * 4 * 256) * 4 <= 160 * 1024;
    static constexpr int TOTAL = XC + (XCH ? kWaves * 4 * 256 : 0);
    static_assert(!GRAD || 32 * NPAD <= 2 * kRows * XP, "bias and gain sums must fit over the x and dy rows");
    static_assert(!GRAD || kRows * N2P <= 2 * kRows * XP, "angle terms must fit over the x and dy rows");
    static_assert(!GRAD || kWaves * 64 <= SLAB, "angle-sum scratch must fit in the slab area");
    static_assert(!(GRAD && SPLIT), "the gradient kernel needs every tile");
    static_assert(TOTAL * 4 <= 160 * 1024, "LDS");
};

// Running angle sums of a chunk: phi[k][i] = theta summed over tokens 0..k of the chunk
// (pairs i >= nr: 0).  The loads are issued by angle_load, the sums by angle_scan
// (scratch: [8][64]).
template <int N2P>
struct AngleTile {
    static constexpr int Q = kRows * N2P / kThreads > 0 ? kRows * N2P / kThreads : 1;
    float v[Q];
};
template <int N2P>
__device__ __forceinline__ void angle_load(const BwdParams &p, AngleTile<N2P> &a, int64_t b, int h, int64_t t0, int Tv) {
    const int tid = threadIdx.x, NR = p.nr;
#pragma unroll
    for (int q = 0; q < AngleTile<N2P>::Q; ++q) {
        const int e = tid + kThreads * q, k = e / N2P, i = e - k * N2P;
        const bool ok = NR > 0 && e < kRows * N2P && k < Tv && i < NR;
        const float v = NR > 0 ? ld_raw(p.theta, ((b * p.T + t0 + k) * p.H + h) * (int64_t)NR + i, ok) : 0.f;
        a.v[q] = ok ? v : 0.f;
    }
}
template <int N2P>
__device__ void angle_scan_lds(float *phi, float *scratch);
template <int N2P>
__device__ void angle_scan(const AngleTile<N2P> &a, float *phi, float *scratch) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < AngleTile<N2P>::Q; ++q) {
        const int e = tid + kThreads * q;
        if (e < kRows * N2P) phi[e] = a.v[q];
    }
    angle_scan_lds<N2P>(phi, scratch);
}
// running sums over the tokens of the angles staged in phi[64][N2P]
template <int N2P>
__device__ void angle_scan_lds(float *phi, float *scratch) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    (void)tid;
    __syncthreads();
    float run = 0.f;
    if (lane < N2P) {
#pragma unroll
        for (int k = 8 * wv; k < 8 * wv + 8; ++k) run += phi[k * N2P + lane];
        scratch[wv * 64 + lane] = run;
    }
    __syncthreads();
    if (lane < N2P) {
        float off = 0.f;
        for (int ww = 0; ww < wv; ++ww) off += scratch[ww * 64 + lane];
#pragma unroll
        for (int k = 8 * wv; k < 8 * wv + 8; ++k) {
            off += phi[k * N2P + lane];
            phi[k * N2P + lane] = off;
        }
    }
    __syncthreads();
}

// 16-byte load of 16 / sizeof(T) consecutive elements (offset 0 when absent)
template <class T>
__device__ __forceinline__ u32x4_t ld_vec(const T *base, int64_t off, bool ok) {
    return *reinterpret_cast<const u32x4_t *>(base + (ok ? off : 0));
}
template <class Io>
__device__ __forceinline__ float vec_elem(const u32x4_t &v, int j) {
    if constexpr (Io::bytes == 2) {
        const uint32_t w = v[j >> 1];
        return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
        return __uint_as_float(v[j]);
    }
}

// The chunk staging of chunk_prologue with 16-byte loads: each (token, rank-interleaved row)
// run of x, dy, z, B and C and each token's angles are read as whole vectors (one or two per
// thread), unpacked into the LDS tiles, and the B and C rows are then normalised and rotated
// in place.  Needs P R and N R multiples of 16 / sizeof(element) and nr a multiple of 4.
// SIDES: 3 stages both sides; 1 (B~ and x, with the per-token scalars, angles and row tables)
// and then 2 (C~ and gated dy, reusing those) stage one side at a time into the shared tiles
// of the split layout.
template <class Io, int NPAD, int PPAD, bool SCALED, int SIDES = 3, bool HS = false>
__device__ float chunk_prologue_vec(const BwdParams &p, float *sm, int64_t b, int h, int64_t t0, int Tv) {
    using ET = typename Io::T;
    using L = CL<NPAD, PPAD, !SCALED, SIDES != 3>;
    constexpr bool DOB = (SIDES & 1) != 0, DOC = (SIDES & 2) != 0;
    constexpr int E = 16 / Io::bytes;
    constexpr int QX = (kRows * PPAD / E + kThreads - 1) / kThreads;
    constexpr int QB = (kRows * NPAD / E + kThreads - 1) / kThreads;
    constexpr int QT = (kRows * L::N2P / 4 + kThreads - 1) / kThreads;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int N = p.N, P = p.P, R = p.R, N2 = N / 2, NR = p.nr;
    const int Qt = kRows / R, rows = Tv * R;
    const int64_t T = p.T, H = p.H;
    float *tk = sm + L::TK, *rt = sm + L::RT, *phi = sm + L::PH;
    // ---- loads
    const int k0 = tid;  // token of the chunk (wave 0)
    const bool okt = tid < 64 && k0 < Tv, okn = okt && t0 + k0 + 1 < T;
    const int64_t btt = (b * T + t0 + k0) * H + h;
    float dtr = ld_raw(p.dt, btt, okt), lmr = ld_raw(p.lam, btt, okt);
    float Ar = (p.flags & kFlagAPerToken) ? ld_raw(p.A, btt, okt) : p.A[h];
    float dtn = ld_raw(p.dt, btt + H, okn), lmn = ld_raw(p.lam, btt + H, okn);
    const int vx = P * R / E, vb = N * R / E, vt = NR / 4;
    const ET *zp = (const ET *)(p.z ? p.z : p.x);
    u32x4_t xv[QX], yv[QX], zv[QX], bv[QB], cv[QB], tv[QT];
#pragma unroll
    for (int q = 0; q < QX; ++q) {
        const int e = tid + kThreads * q, k = e / vx, v = e - k * vx;
        const bool ok = e < Tv * vx;
        const int64_t o = ((b * T + t0 + k) * H + h) * (int64_t)P * R + (int64_t)v * E;
        xv[q] = ld_vec((const ET *)p.x, o, ok);
        yv[q] = ld_vec((const ET *)p.dy, o, ok);
        zv[q] = ld_vec(zp, o, ok);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        const int e = tid + kThreads * q, k = e / vb, v = e - k * vb;
        const bool ok = e < Tv * vb;
        const int64_t o = ((b * T + t0 + k) * H + h) * (int64_t)N * R + (int64_t)v * E;
        bv[q] = ld_vec((const ET *)p.Bm, o, ok);
        cv[q] = ld_vec((const ET *)p.Cm, o, ok);
    }
#pragma unroll
    for (int q = 0; q < QT; ++q) {
        const int e = tid + kThreads * q, k = vt > 0 ? e / vt : 0, v = e - k * vt;
        const bool ok = vt > 0 && e < Tv * vt;
        tv[q] = ld_vec(p.theta ? p.theta : p.dt, ((b * T + t0 + k) * H + h) * (int64_t)NR + 4 * v, ok);
    }
    // gains and (rank wv % R when R divides 8) biases of this lane's pair
    using RP = RowPass<L::N2P>;
    const int pl = RP::pair();
    const float *bnp = p.bnw ? p.bnw : p.dt, *cnp = p.cnw ? p.cnw : p.dt;
    const bool okg = pl < N2;
    const int q0 = pc0<HS, NPAD>(pl), q1 = pc1<HS, NPAD>(pl);  // this lane's two columns
    float gb0 = ld_raw(bnp, q0, okg && p.bnw), gb1 = ld_raw(bnp, q1, okg && p.bnw);
    float gc0 = ld_raw(cnp, q0, okg && p.cnw), gc1 = ld_raw(cnp, q1, okg && p.cnw);
    const bool rdiv = (8 % R) == 0;
    const float *bbp = p.bbias ? p.bbias : p.dt, *cbp = p.cbias ? p.cbias : p.dt;
    const int64_t obw = ((int64_t)h * R + (wv % R)) * N;
    float bw0 = ld_raw(bbp, obw + q0, okg && rdiv && p.bbias), bw1 = ld_raw(bbp, obw + q1, okg && rdiv && p.bbias);
    float cw0 = ld_raw(cbp, obw + q0, okg && rdiv && p.cbias), cw1 = ld_raw(cbp, obw + q1, okg && rdiv && p.cbias);
    // ---- zero padding of the tiles (disjoint from the loaded elements)
    for (int row = wv; row < kRows; row += kWaves) {
        for (int col = lane; col < L::XP; col += 64)
            if (row >= rows || col >= P) {
                if (DOB) sm[L::SX + row * L::XP + col] = 0.f;
                if (DOC) sm[L::SY + row * L::XP + col] = 0.f;
            }
        for (int col = lane; col < L::BP; col += 64)
            if (row >= rows || col >= N) {
                if (DOB) sm[L::SB + row * L::BP + col] = 0.f;
                if (DOC) sm[L::SC + row * L::BP + col] = 0.f;
            }
        if (DOB && lane < L::N2P && (row >= Tv || lane >= NR)) phi[row * L::N2P + lane] = 0.f;
    }
    // ---- per-token scalars (wave 0; lane = token of the chunk)
    if (DOB && tid < 64) {
        float la = 0.f, kap = 0.f, gam = 0.f;
        if (k0 < Tv) {
            float dt = dtr, lam = lmr, dn = dtn, ln = lmn;
            if (p.flags & kFlagDtSoftplus) {
                const float bias = p.dtbias ? p.dtbias[h] : 0.f;
                dt = softplus_f(dt + bias);
                dn = softplus_f(dn + bias);
            }
            if (p.flags & kFlagLamSigmoid) {
                lam = sigmoid_f(lam);
                ln = sigmoid_f(ln);
            }
            la = dt * Ar;
            gam = lam * dt;
            kap = gam + (okn ? dn * (1.f - ln) : 0.f);
        }
        const float cs = wave_incl_scan(la);
        tk[k0] = cs;
        tk[64 + k0] = kap;
        tk[128 + k0] = gam;
    }
    // ---- unpack x, gated dy, raw B and C, angles
    float dDp = 0.f;
#pragma unroll
    for (int q = 0; q < QX; ++q) {
        const int e = tid + kThreads * q, k = e / vx, v = e - k * vx;
        if (e >= Tv * vx) continue;
        int pc = (v * E) / R, r = v * E - pc * R;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const float xf = vec_elem<Io>(xv[q], j);
            float yf = vec_elem<Io>(yv[q], j);
            if (DOC && p.z) yf *= silu_f(vec_elem<Io>(zv[q], j));
            if (DOB) sm[L::SX + (k * R + r) * L::XP + pc] = xf;
            if (DOC) sm[L::SY + (k * R + r) * L::XP + pc] = yf;
            if (DOB && DOC) dDp += xf * yf;
            if (++r == R) {
                r = 0;
                ++pc;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        const int e = tid + kThreads * q, k = e / vb, v = e - k * vb;
        if (e >= Tv * vb) continue;
        int n = (v * E) / R, r = v * E - n * R;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if (DOB) sm[L::SB + (k * R + r) * L::BP + n] = vec_elem<Io>(bv[q], j);
            if (DOC) sm[L::SC + (k * R + r) * L::BP + n] = vec_elem<Io>(cv[q], j);
            if (++r == R) {
                r = 0;
                ++n;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < QT; ++q) {
        const int e = tid + kThreads * q, k = vt > 0 ? e / vt : 0, v = e - k * vt;
        if (!DOB || vt == 0 || e >= Tv * vt) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) phi[k * L::N2P + 4 * v + j] = __uint_as_float(tv[q][j]);
    }
    if constexpr (DOB) angle_scan_lds<L::N2P>(phi, sm + L::RW);  // (its barriers publish every tile and tk)
    else __syncthreads();                                          // (the tiles; tk and rt are staged)
    const float cs_end = tk[Tv - 1];
    if (DOB && tid < kRows) {
        const int rho = tid, k = rho / R;
        const bool valid = k < Qt && k < Tv;
        const float cs = valid ? tk[k] : cs_end;
        rt[rho] = cs;
        rt[64 + rho] = valid ? tk[64 + k] : 0.f;
        rt[128 + rho] = valid ? tk[128 + k] : 0.f;
        rt[192 + rho] = __int_as_float(valid ? k : 1 << 20);
        rt[256 + rho] = __expf(cs_end - cs);
        rt[320 + rho] = __expf(cs);
    }
    __syncthreads();  // row tables
    // ---- B and C rows in place: norm, gain, bias, rotation (and scale); lane = pair
    const bool norm = (p.flags & kFlagNorm) != 0;
    const float invN = 1.f / (float)N;
    gb0 = okg && p.bnw ? gb0 : 1.f;
    gb1 = okg && p.bnw ? gb1 : 1.f;
    gc0 = okg && p.cnw ? gc0 : 1.f;
    gc1 = okg && p.cnw ? gc1 : 1.f;
    const int lp = pl < L::N2P ? pl : 0;
    const int l0 = pc0<HS, NPAD>(lp), l1 = pc1<HS, NPAD>(lp);  // the clamped pair's columns, for the LDS reads
#pragma unroll
    for (int m = 0; m < RP::NM; ++m) {
        const int rho = RP::row(wv, m), k = rho / R, r = rho - k * R;
        const bool valid = k < Qt && k < Tv && pl < N2;
        float b0 = DOB ? sm[L::SB + rho * L::BP + l0] : 0.f, b1 = DOB ? sm[L::SB + rho * L::BP + l1] : 0.f;
        float c0 = DOC ? sm[L::SC + rho * L::BP + l0] : 0.f, c1 = DOC ? sm[L::SC + rho * L::BP + l1] : 0.f;
        b0 = valid ? b0 : 0.f;
        b1 = valid ? b1 : 0.f;
        c0 = valid ? c0 : 0.f;
        c1 = valid ? c1 : 0.f;
        float sb = 1.f, sc = 1.f;
        if (norm) {
            if (DOB) sb = rsqrtf(RP::sum(b0 * b0 + b1 * b1) * invN + p.eps);
            if (DOC) sc = rsqrtf(RP::sum(c0 * c0 + c1 * c1) * invN + p.eps);
            if (L::KEEP && pl == 0) {
                sm[L::RS + rho] = sb;
                sm[L::RS + 64 + rho] = sc;
            }
        }
        float bi0 = bw0, bi1 = bw1, ci0 = cw0, ci1 = cw1;
        if (!rdiv) {
            const int64_t ob = ((int64_t)h * R + r) * N;
            if (DOB) {
                bi0 = ld_raw(bbp, ob + q0, valid && p.bbias);
                bi1 = ld_raw(bbp, ob + q1, valid && p.bbias);
            }
            if (DOC) {
                ci0 = ld_raw(cbp, ob + q0, valid && p.cbias);
                ci1 = ld_raw(cbp, ob + q1, valid && p.cbias);
            }
        }
        bi0 = p.bbias ? bi0 : 0.f;
        bi1 = p.bbias ? bi1 : 0.f;
        ci0 = p.cbias ? ci0 : 0.f;
        ci1 = p.cbias ? ci1 : 0.f;
        b0 = (norm ? b0 * sb * gb0 : b0) + bi0;
        b1 = (norm ? b1 * sb * gb1 : b1) + bi1;
        c0 = (norm ? c0 * sc * gc0 : c0) + ci0;
        c1 = (norm ? c1 * sc * gc1 : c1) + ci1;
        float sn, cn;
        fast_sincos(phi[(k < kRows ? k : 0) * L::N2P + lp], sn, cn);
        float fb = 1.f, fc = 1.f;
        if (SCALED) {
            fb = rt[256 + rho] * rt[64 + rho];
            fc = rt[320 + rho];
        }
        const float u0 = fb * (cn * b0 - sn * b1), u1 = fb * (sn * b0 + cn * b1);
        const float v0 = fc * (cn * c0 - sn * c1), v1 = fc * (sn * c0 + cn * c1);
        if (pl < L::N2P) {
            if (DOB) {
                sm[L::SB + rho * L::BP + q0] = valid ? u0 : 0.f;
                sm[L::SB + rho * L::BP + q1] = valid ? u1 : 0.f;
            }
            if (DOC) {
                sm[L::SC + rho * L::BP + q0] = valid ? v0 : 0.f;
                sm[L::SC + rho * L::BP + q1] = valid ? v1 : 0.f;
            }
        }
    }
    __syncthreads();
    return dDp;
}

// Stage one chunk: per-token scalars, normalised + biased + rotated B and C rows (scaled by
// e^(cs_end - cs) kappa and e^cs when SCALED), x and gated dy rows, zero padding.  Every
// global load of the chunk is issued before the first use.
// Returns (per thread) its part of sum(dy_gated * x).  SIDES as in chunk_prologue_vec.
template <class Io, int NPAD, int PPAD, bool SCALED, int SIDES = 3, bool HS = false>
__device__ float chunk_prologue(const BwdParams &p, float *sm, int64_t b, int h, int64_t t0, int Tv) {
    using ET = typename Io::T;
    using L = CL<NPAD, PPAD, !SCALED, SIDES != 3>;
    constexpr bool DOB = (SIDES & 1) != 0, DOC = (SIDES & 2) != 0;
    constexpr int QX = kRows * PPAD / kThreads;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int N = p.N, P = p.P, R = p.R, N2 = N / 2;
    const int Qt = kRows / R;
    const int64_t T = p.T, H = p.H;
    float *tk = sm + L::TK, *rt = sm + L::RT;
    // ---- loads
    const int k0 = tid;  // token of the chunk (wave 0)
    const bool okt = tid < 64 && k0 < Tv, okn = okt && t0 + k0 + 1 < T;
    const int64_t btt = (b * T + t0 + k0) * H + h;
    float dtr = ld_raw(p.dt, btt, okt), lmr = ld_raw(p.lam, btt, okt);
    float Ar = (p.flags & kFlagAPerToken) ? ld_raw(p.A, btt, okt) : p.A[h];
    float dtn = ld_raw(p.dt, btt + H, okn), lmn = ld_raw(p.lam, btt + H, okn);
    AngleTile<L::N2P> ang;
    angle_load<L::N2P>(p, ang, b, h, t0, Tv);
    ET xr[QX], yr[QX], zr[QX];
    bool xo[QX];
    const int nx = Qt * PPAD * R;
    const ET *zp = (const ET *)(p.z ? p.z : p.x);
#pragma unroll
    for (int q = 0; q < QX; ++q) {
        const int e = tid + kThreads * q;
        const int k = e / (PPAD * R), rem = e - k * PPAD * R, pc = rem / R, r = rem - pc * R;
        xo[q] = e < nx && k < Tv && pc < P;
        const int64_t o = ((b * T + t0 + k) * H + h) * (int64_t)P * R + (int64_t)pc * R + r;
        xr[q] = ld_raw((const ET *)p.x, o, xo[q]);
        yr[q] = ld_raw((const ET *)p.dy, o, xo[q]);
        zr[q] = ld_raw(zp, o, xo[q]);
    }
    using RP = RowPass<L::N2P>;
    constexpr int NM = RP::NM;
    const int pl = RP::pair();
    const int q0 = pc0<HS, NPAD>(pl), q1 = pc1<HS, NPAD>(pl);  // this lane's two columns
    ET rbr[NM][2], rcr[NM][2];
    float bb[NM][2], cb[NM][2];
    bool ro[NM];
    const float *bbp = p.bbias ? p.bbias : p.dt, *cbp = p.cbias ? p.cbias : p.dt;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int rho = RP::row(wv, m), k = rho / R, r = rho - k * R;
        ro[m] = k < Qt && k < Tv && pl < N2;
        const int64_t o = ((b * T + t0 + k) * H + h) * (int64_t)N * R + r;
        rbr[m][0] = ld_raw((const ET *)p.Bm, o + (int64_t)q0 * R, ro[m]);
        rbr[m][1] = ld_raw((const ET *)p.Bm, o + (int64_t)q1 * R, ro[m]);
        rcr[m][0] = ld_raw((const ET *)p.Cm, o + (int64_t)q0 * R, ro[m]);
        rcr[m][1] = ld_raw((const ET *)p.Cm, o + (int64_t)q1 * R, ro[m]);
        const int64_t ob = ((int64_t)h * R + r) * N;
        bb[m][0] = ld_raw(bbp, ob + q0, ro[m] && p.bbias);
        bb[m][1] = ld_raw(bbp, ob + q1, ro[m] && p.bbias);
        cb[m][0] = ld_raw(cbp, ob + q0, ro[m] && p.cbias);
        cb[m][1] = ld_raw(cbp, ob + q1, ro[m] && p.cbias);
    }
    const float *bnp = p.bnw ? p.bnw : p.dt, *cnp = p.cnw ? p.cnw : p.dt;
    const bool okg = pl < N2;
    float gb0 = ld_raw(bnp, q0, okg && p.bnw), gb1 = ld_raw(bnp, q1, okg && p.bnw);
    float gc0 = ld_raw(cnp, q0, okg && p.cnw), gc1 = ld_raw(cnp, q1, okg && p.cnw);
    // ---- values (after every load is in flight)
    dtr = okt ? dtr : 0.f;
    lmr = okt ? lmr : 0.f;
    Ar = okt ? Ar : 0.f;
    dtn = okn ? dtn : 0.f;
    lmn = okn ? lmn : 0.f;
    gb0 = okg && p.bnw ? gb0 : 1.f;
    gb1 = okg && p.bnw ? gb1 : 1.f;
    gc0 = okg && p.cnw ? gc0 : 1.f;
    gc1 = okg && p.cnw ? gc1 : 1.f;
    float rb[NM][2], rc[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            rb[m][j] = raw_f<Io>(rbr[m][j], ro[m]);
            rc[m][j] = raw_f<Io>(rcr[m][j], ro[m]);
            bb[m][j] = ro[m] && p.bbias ? bb[m][j] : 0.f;
            cb[m][j] = ro[m] && p.cbias ? cb[m][j] : 0.f;
        }
    }
    // ---- per-token scalars (wave 0; lane = token of the chunk)
    if (DOB && tid < 64) {
        float la = 0.f, kap = 0.f, gam = 0.f;
        if (k0 < Tv) {
            float dt = dtr, lam = lmr, dn = dtn, ln = lmn;
            if (p.flags & kFlagDtSoftplus) {
                const float bias = p.dtbias ? p.dtbias[h] : 0.f;
                dt = softplus_f(dt + bias);
                dn = softplus_f(dn + bias);
            }
            if (p.flags & kFlagLamSigmoid) {
                lam = sigmoid_f(lam);
                ln = sigmoid_f(ln);
            }
            la = dt * Ar;
            gam = lam * dt;
            kap = gam + (t0 + k0 + 1 < T ? dn * (1.f - ln) : 0.f);
        }
        const float cs = wave_incl_scan(la);
        tk[k0] = cs;
        tk[64 + k0] = kap;
        tk[128 + k0] = gam;
    }
    // ---- x and gated dy rows
    float dDp = 0.f;
#pragma unroll
    for (int q = 0; q < QX; ++q) {
        const int e = tid + kThreads * q;
        if (e >= nx) continue;
        const int k = e / (PPAD * R), rem = e - k * PPAD * R, pc = rem / R, r = rem - pc * R;
        const float xv = raw_f<Io>(xr[q], xo[q]), yv = raw_f<Io>(yr[q], xo[q]);
        const float y = (DOC && p.z) ? yv * silu_f(raw_f<Io>(zr[q], xo[q])) : yv;
        if (DOB) sm[L::SX + (k * R + r) * L::XP + pc] = xv;
        if (DOC) sm[L::SY + (k * R + r) * L::XP + pc] = y;
        if (DOB && DOC) dDp += xv * y;
    }
    for (int e = tid; e < (kRows - Qt * R) * L::XP; e += kThreads) {
        if (DOB) sm[L::SX + Qt * R * L::XP + e] = 0.f;
        if (DOC) sm[L::SY + Qt * R * L::XP + e] = 0.f;
    }
    if constexpr (DOB) angle_scan<L::N2P>(ang, sm + L::PH, sm + L::RW);  // (its barriers publish tk)
    else __syncthreads();
    const float cs_end = tk[Tv - 1];
    // per-row tables
    if (DOB && tid < kRows) {
        const int rho = tid, k = rho / R;
        const bool valid = k < Qt && k < Tv;
        const float cs = valid ? tk[k] : cs_end;
        rt[rho] = cs;
        rt[64 + rho] = valid ? tk[64 + k] : 0.f;
        rt[128 + rho] = valid ? tk[128 + k] : 0.f;
        rt[192 + rho] = __int_as_float(valid ? k : 1 << 20);
        rt[256 + rho] = __expf(cs_end - cs);
        rt[320 + rho] = __expf(cs);
    }
    __syncthreads();  // row tables
    // B and C rows: wave wv takes rows wv + 8 m; lane = pair.  Branch-free (absent lanes and
    // rows compute on zeros and are masked at the store) so that the rows' reductions overlap.
    const bool norm = (p.flags & kFlagNorm) != 0;
    const float invN = 1.f / (float)N;
    const float *phi = sm + L::PH;
    const int lp = pl < L::N2P ? pl : 0;  // clamped pair for the LDS reads
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int rho = RP::row(wv, m), k = rho / R;
        const bool valid = ro[m];
        const int kc = k < kRows ? k : 0;
        float sb = 1.f, sc = 1.f;
        if (norm) {
            if (DOB) sb = rsqrtf(RP::sum(rb[m][0] * rb[m][0] + rb[m][1] * rb[m][1]) * invN + p.eps);
            if (DOC) sc = rsqrtf(RP::sum(rc[m][0] * rc[m][0] + rc[m][1] * rc[m][1]) * invN + p.eps);
            if (L::KEEP && pl == 0) {
                sm[L::RS + rho] = sb;
                sm[L::RS + 64 + rho] = sc;
            }
        }
        float b0 = (norm ? rb[m][0] * sb * gb0 : rb[m][0]) + bb[m][0];
        float b1 = (norm ? rb[m][1] * sb * gb1 : rb[m][1]) + bb[m][1];
        float c0 = (norm ? rc[m][0] * sc * gc0 : rc[m][0]) + cb[m][0];
        float c1 = (norm ? rc[m][1] * sc * gc1 : rc[m][1]) + cb[m][1];
        float sn, cn;
        fast_sincos(phi[kc * L::N2P + lp], sn, cn);
        float fb = 1.f, fc = 1.f;
        if (SCALED) {
            fb = rt[256 + rho] * rt[64 + rho];
            fc = rt[320 + rho];
        }
        const float u0 = fb * (cn * b0 - sn * b1), u1 = fb * (sn * b0 + cn * b1);
        const float v0 = fc * (cn * c0 - sn * c1), v1 = fc * (sn * c0 + cn * c1);
        if (pl < L::N2P) {
            if (DOB) {
                sm[L::SB + rho * L::BP + q0] = valid ? u0 : 0.f;
                sm[L::SB + rho * L::BP + q1] = valid ? u1 : 0.f;
            }
            if (DOC) {
                sm[L::SC + rho * L::BP + q0] = valid ? v0 : 0.f;
                sm[L::SC + rho * L::BP + q1] = valid ? v1 : 0.f;
            }
        }
    }
    __syncthreads();
    return dDp;
}

__device__ __forceinline__ float block_sum(float v, float *scratch) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) scratch[wv] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += scratch[w];
    return s;
}

}  // namespace

// ---------------------------------------------------------------- per-chunk state sums
// On the 16-byte load path, a layout that leaves room for only one workgroup per compute unit
// stages one side at a time (B~ and x, then C~ and dy) when that makes room for two; the
// register budget then follows two workgroups per unit (the launch bound counts waves per SIMD).
template <int NPAD, int PPAD, bool VEC>
constexpr bool state_split() {
    return VEC && CL<NPAD, PPAD>::TOTAL * 4 * 2 > 160 * 1024 && CL<NPAD, PPAD, false, true>::TOTAL * 4 * 2 <= 160 * 1024;
}
template <int NPAD, int PPAD, bool VEC>
constexpr int state_min_waves_per_simd() { return state_split<NPAD, PPAD, VEC>() ? 2 * kThreads / 256 : 1; }

template <class Io, int NPAD, int PPAD, bool VEC, bool HS = false>
__global__ __launch_bounds__(kThreads, (state_min_waves_per_simd<NPAD, PPAD, VEC>())) void bwd_chunk_state_kernel(BwdParams p) {
    constexpr bool SPLIT = state_split<NPAD, PPAD, VEC>();
    using L = CL<NPAD, PPAD, false, SPLIT>;
    constexpr int NT = NPAD / 16, PT = PPAD / 16;
    extern __shared__ __attribute__((aligned(16))) float sm[];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, l16 = lane & 15;
    const int nck = p.nck, N = p.N, P = p.P, N2 = N / 2;
    const int64_t bh = blockIdx.x / nck;
    const int c = (int)(blockIdx.x - bh * nck);
    M3_DCHECK(p, bh < p.B * p.H && c < nck && (int64_t)c * (kRows / p.R) < p.T);
    const int64_t b = bh / p.H;
    const int h = (int)(bh - b * p.H);
    const int Qt = kRows / p.R;
    const int64_t t0 = (int64_t)c * Qt;
    const int Tv = (int)min((int64_t)Qt, p.T - t0);
    const int64_t cidx = bh * nck + c;
    // S (which 0) = sum over rows of B~ x^T, U (which 1) = sum of C~ dy^T: this wave's 16x16 tiles
    auto products = [&](int which, int q0, int q1) {
        for (int q = q0 + wv; q < q1; q += kWaves) {
            const int rem = q - which * NT * PT, a = rem / PT, bq = rem - a * PT;
            const float *Ao = sm + (which ? L::SC : L::SB), *Bo = sm + (which ? L::SY : L::SX);
            f32x4_t acc = zero4();
#pragma unroll
            for (int kc = 0; kc < kRows / 32; ++kc) {
                float av[8], bv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = 32 * kc + 8 * g + j;
                    av[j] = Ao[s * L::BP + 16 * a + l16];
                    bv[j] = Bo[s * L::XP + 16 * bq + l16];
                }
                acc = mma8(av, bv, acc);
            }
            float *dst = (which ? p.Ust : p.Sst) + cidx * N * (int64_t)P;
            const int pc = 16 * bq + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 16 * a + 4 * g + i;
                if (n < N && pc < P) dst[(int64_t)n * P + pc] = acc[i];
            }
        }
    };
    if constexpr (SPLIT) {
        if constexpr (VEC) chunk_prologue_vec<Io, NPAD, PPAD, true, 1, HS>(p, sm, b, h, t0, Tv);
        else chunk_prologue<Io, NPAD, PPAD, true, 1, HS>(p, sm, b, h, t0, Tv);
        products(0, 0, NT * PT);
        __syncthreads();  // the shared tiles are restaged for the C side
        if constexpr (VEC) chunk_prologue_vec<Io, NPAD, PPAD, true, 2, HS>(p, sm, b, h, t0, Tv);
        else chunk_prologue<Io, NPAD, PPAD, true, 2, HS>(p, sm, b, h, t0, Tv);
        products(1, NT * PT, 2 * NT * PT);
    } else {
        if constexpr (VEC) chunk_prologue_vec<Io, NPAD, PPAD, true, 3, HS>(p, sm, b, h, t0, Tv);
        else chunk_prologue<Io, NPAD, PPAD, true, 3, HS>(p, sm, b, h, t0, Tv);
        products(0, 0, NT * PT);
        products(1, NT * PT, 2 * NT * PT);
    }
    if (tid < N2) p.phic[cidx * N2 + tid] = sm[L::PH + (Tv - 1) * L::N2P + tid];
    if (tid == 0) p.lsum[cidx] = sm[L::TK + Tv - 1];
}

// ---------------------------------------------------------------- state passes over the chunks
// blockIdx.y 0: states before each chunk (in place of S); 1: adjoints after each chunk (in
// place of U) and the initial state's adjoint.  Thread: (sequence, pair, column).  Each
// thread's chain over the chunks is serial; the loads of KQ chunks are issued together (8 or
// 16 measured slower at T 16384: the registers they take halve the waves in flight).
__global__ __launch_bounds__(256) void bwd_state_pass_kernel(BwdParams p) {
    constexpr int KQ = 4;
    const int N = p.N, P = p.P, N2 = N / 2, NR = p.nr, R = p.R, nck = p.nck;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= p.B * p.H * N2 * (int64_t)P) return;
    const int pc = (int)(e % P);
    const int i = (int)((e / P) % N2);
    const int64_t bh = e / ((int64_t)P * N2);
    const int64_t b = bh / p.H;
    const int h = (int)(bh - b * p.H);
    const bool rot = i < NR;
    const int64_t NP = (int64_t)N * P;
    const int n0 = pn0(p, i), n1 = pn1(p, i);        // the pair's two state rows
    const int64_t dr = (int64_t)(n1 - n0) * P;        // from the first row to the second
    if (blockIdx.y == 0) {
        float g0 = 0.f, g1 = 0.f;
        if (p.h0) {
            g0 = p.h0[(bh * N + n0) * P + pc];
            g1 = p.h0[(bh * N + n1) * P + pc];
        }
        if (p.pB0 && p.px0) {
            const float eta = eta_at(p, b, h, -1);
            float a0 = 0.f, a1 = 0.f;
            for (int r = 0; r < R; ++r) {
                const float xv = p.px0[(bh * P + pc) * R + r];
                a0 += p.pB0[(bh * N + n0) * R + r] * xv;
                a1 += p.pB0[(bh * N + n1) * R + r] * xv;
            }
            g0 += eta * a0;
            g1 += eta * a1;
        }
        if (rot && p.ang0) {
            float s, c;
            fast_sincos((float)wrap_2pi((double)p.ang0[bh * NR + i]), s, c);
            const float u = c * g0 + s * g1, v = -s * g0 + c * g1;
            g0 = u;
            g1 = v;
        }
        float *S = p.Sst + bh * nck * NP + (int64_t)n0 * P + pc;
        for (int c0 = 0; c0 < nck; c0 += KQ) {
            float s0[KQ], s1[KQ], dec[KQ], ph[KQ];
#pragma unroll
            for (int q = 0; q < KQ; ++q) {
                const int ck = c0 + q;
                s0[q] = s1[q] = ph[q] = dec[q] = 0.f;
                if (ck < nck) {
                    s0[q] = S[ck * NP];
                    s1[q] = S[ck * NP + dr];
                    dec[q] = p.lsum[bh * nck + ck];
                    ph[q] = rot ? p.phic[(bh * nck + ck) * N2 + i] : 0.f;
                }
            }
#pragma unroll
            for (int q = 0; q < KQ; ++q) {
                const int ck = c0 + q;
                if (ck < nck) {
                    S[ck * NP] = g0;
                    S[ck * NP + dr] = g1;
                    const float d = __expf(dec[q]);
                    const float u = d * g0 + s0[q], v = d * g1 + s1[q];
                    if (ck == nck - 1) {  // state after the last chunk, in its frame
                        p.hfin[(bh * N + n0) * P + pc] = u;
                        p.hfin[(bh * N + n1) * P + pc] = v;
                    } else {
                        float s, c;
                        fast_sincos(ph[q], s, c);
                        g0 = c * u + s * v;
                        g1 = -s * u + c * v;
                    }
                }
            }
        }
        return;
    }
    // reverse: the frame of the last chunk is the angle before it
    double th = (rot && p.ang0) ? (double)p.ang0[bh * NR + i] : 0.0;
    if (rot)
        for (int c0 = 0; c0 + 1 < nck; c0 += KQ) {
            float v[KQ];  // KQ independent loads in flight, summed in chunk order
#pragma unroll
            for (int q = 0; q < KQ; ++q) v[q] = c0 + q + 1 < nck ? p.phic[(bh * nck + c0 + q) * N2 + i] : 0.f;
#pragma unroll
            for (int q = 0; q < KQ; ++q) th += (double)v[q];
        }
    const float thl = rot ? (float)wrap_2pi(th) : 0.f;
    if (pc == 0) p.thst[bh * N2 + i] = thl;
    float gb0 = 0.f, gb1 = 0.f;
    if (p.dh1) {
        const float d0 = p.dh1[(bh * N + n0) * P + pc], d1 = p.dh1[(bh * N + n1) * P + pc];
        float s = 0.f, c = 1.f;
        if (rot) fast_sincos(thl, s, c);
        gb0 = c * d0 + s * d1;
        gb1 = -s * d0 + c * d1;
    }
    float *U = p.Ust + bh * nck * NP + (int64_t)n0 * P + pc;
    for (int c0 = nck - 1; c0 >= 0; c0 -= KQ) {
        float u0[KQ], u1[KQ], dec[KQ], ph[KQ];
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            const int ck = c0 - q;
            u0[q] = u1[q] = ph[q] = dec[q] = 0.f;
            if (ck >= 0) {
                u0[q] = U[ck * NP];
                u1[q] = U[ck * NP + dr];
                dec[q] = p.lsum[bh * nck + ck];
                ph[q] = (rot && ck > 0) ? p.phic[(bh * nck + ck - 1) * N2 + i] : 0.f;
            }
        }
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            const int ck = c0 - q;
            if (ck >= 0) {
                U[ck * NP] = gb0;
                U[ck * NP + dr] = gb1;
                const float d = __expf(dec[q]);
                const float a = d * gb0 + u0[q], v = d * gb1 + u1[q];
                float s, c;
                fast_sincos(ph[q], s, c);
                gb0 = c * a - s * v;
                gb1 = s * a + c * v;
            }
        }
    }
    // adjoint of the state before the first chunk, in the global frame
    float s = 0.f, c = 1.f;
    if (rot && p.ang0) fast_sincos((float)wrap_2pi((double)p.ang0[bh * NR + i]), s, c);
    p.G0w[(bh * N + n0) * P + pc] = c * gb0 - s * gb1;
    p.G0w[(bh * N + n1) * P + pc] = s * gb0 + c * gb1;
}

// ---------------------------------------------------------------- per-chunk gradients
// HS: the half-split pairing (p.hs, N = NPAD of 64 or 128), compiled separately so that the
// adjacent pairing's per-column angle terms keep their lane-pair form.
template <class Io, int NPAD, int PPAD, bool HS = false>
__global__ __launch_bounds__(kThreads) void bwd_chunk_grad_kernel(BwdParams p) {
    using ET = typename Io::T;
    using L = CL<NPAD, PPAD, true>;
    constexpr int NT = NPAD / 16, PT = PPAD / 16, NH = NT / 2, PH = PT / 2, NS = NPAD / 32;
    constexpr int BP = L::BP, XP = L::XP, N2P = L::N2P;
    constexpr int SQ = 32 * PPAD / kThreads;  // slab elements per thread
    extern __shared__ __attribute__((aligned(16))) float sm[];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, l16 = lane & 15;
    // wave (row tile w, column half hf); SIMD wv & 3 hosts row tiles w and 3 - w, which
    // balances the triangular work
    const int hf = wv >> 2, w = hf == 0 ? (wv & 3) : 3 - (wv & 3);
    const int nck = p.nck, N = p.N, P = p.P, R = p.R, N2 = N / 2, NR = p.nr;
    const int64_t bh = blockIdx.x / nck;
    const int c = (int)(blockIdx.x - bh * nck);
    const int64_t b = bh / p.H;
    const int h = (int)(bh - b * p.H);
    const int Qt = kRows / R;
    // row tiles that can hold a nonzero of row tile w: every later tile, and, when a token's
    // rows can straddle two tiles (R not dividing 16), the neighbouring earlier one
    const int st = (16 % R) != 0 ? 1 : 0, amin = w - st, amax = w + st;
    const int64_t T = p.T, H = p.H;
    const int64_t t0 = (int64_t)c * Qt;
    const int Tv = (int)min((int64_t)Qt, T - t0);
    const int64_t cidx = bh * nck + c;
    M3_DCHECK(p, bh < p.B * p.H && c < nck && Tv >= 1 && Tv <= Qt && t0 + Tv <= T);
    const bool last = c == nck - 1;
    const float *Gend = p.Ust + cidx * N * (int64_t)P, *Hst = p.Sst + cidx * N * (int64_t)P;
    // State slabs (32 state rows of the adjoint after the chunk and of the state before it) go
    // through registers into LDS.  The first is loaded before the staging; when the registers
    // allow, every other slab is loaded right after it (in flight during the triangles),
    // otherwise one slab ahead inside the slab loop.  Raw values; masked where they are used.
    constexpr bool PFA = 2 * NS * SQ <= 32 && !(PPAD == 128 && NPAD >= 64);
    float stg[PFA ? 2 * NS : 1][SQ];
    auto slab_ok = [&](int ns, int q) {
        const int e = tid + kThreads * q, row = e / PPAD, col = e - row * PPAD;
        return 32 * ns + row < N && col < P;
    };
    auto load_slab = [&](float (&dst)[SQ], const float *src, int ns) {
#pragma unroll
        for (int q = 0; q < SQ; ++q) {
            const int e = tid + kThreads * q, row = e / PPAD, col = e - row * PPAD;
            dst[q] = ld_raw(src, (int64_t)(32 * ns + row) * P + col, slab_ok(ns, q));
        }
    };
    load_slab(stg[0], Gend, 0);
    // (a run-time choice here: with both staging variants in one kernel the register
    // allocation of the matrix phases comes out better than with either alone)
    const float dDp = p.vec ? chunk_prologue_vec<Io, NPAD, PPAD, false, 3, HS>(p, sm, b, h, t0, Tv)
                            : chunk_prologue<Io, NPAD, PPAD, false, 3, HS>(p, sm, b, h, t0, Tv);
    if constexpr (PFA) {
        load_slab(stg[1], Hst, 0);
#pragma unroll
        for (int ns = 1; ns < NS; ++ns) {
            load_slab(stg[2 * ns], Gend, ns);
            load_slab(stg[2 * ns + 1], Hst, ns);
        }
    }
    float *sB = sm + L::SB, *sC = sm + L::SC, *sX = sm + L::SX, *sY = sm + L::SY, *sS = sm + L::SS;
    const float *rt = sm + L::RT;
    auto rcs = [&](int r) { return rt[r]; };
    auto rkap = [&](int r) { return rt[64 + r]; };
    auto rgam = [&](int r) { return rt[128 + r]; };
    auto rtok = [&](int r) { return __float_as_int(rt[192 + r]); };
    auto rdec = [&](int r) { return rt[256 + r]; };
    auto recs = [&](int r) { return rt[320 + r]; };

    // ------------------------------------------------ s-oriented triangle: P1 = L o G, P2 = L o dY X^T
    // lane value [a][i]: t = 16 a + 4 g + i, s = 16 w + l16 (tiles a < amin are zero)
    f32x4_t P1s[4], P2s[4];
    {
        const int s = 16 * w + l16;
        const float cs_s = rcs(s), kap_s = rkap(s);
        const int tok_s = rtok(s);
        float ce = 0.f;
        // G^T and (dY X^T)^T tiles of this row tile: with the exchange area, wave hf = 0 computes
        // the G tiles and wave hf = 1 the dY X^T tiles, and each reads the other's from LDS;
        // otherwise both waves compute both
        f32x4_t mine[4];
        if constexpr (L::XCH) {
            float *xc = sm + L::XC;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                mine[a] = zero4();
                if (a < amin) continue;
                if (hf == 0) {
#pragma unroll
                    for (int kc = 0; kc < NPAD / 32; ++kc) {
                        float av[8], bv[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            av[j] = sC[(16 * a + l16) * BP + 32 * kc + 8 * g + j];
                            bv[j] = sB[s * BP + 32 * kc + 8 * g + j];
                        }
                        mine[a] = mma8(av, bv, mine[a]);
                    }
                } else {
#pragma unroll
                    for (int kc = 0; kc < PPAD / 32; ++kc) {
                        float av[8], bv[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            av[j] = sY[(16 * a + l16) * XP + 32 * kc + 8 * g + j];
                            bv[j] = sX[s * XP + 32 * kc + 8 * g + j];
                        }
                        mine[a] = mma8(av, bv, mine[a]);
                    }
                }
                *(f32x4_t *)(xc + ((wv * 4 + a) * 64 + lane) * 4) = mine[a];
            }
            __syncthreads();
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            P1s[a] = P2s[a] = zero4();
            float rw[4] = {0.f, 0.f, 0.f, 0.f}, rd[4] = {0.f, 0.f, 0.f, 0.f};
            if (a >= amin) {
                f32x4_t ga = zero4(), da = zero4();
                if constexpr (L::XCH) {
                    // the partner wave (same row tile, other half) is wave 7 - wv
                    const f32x4_t theirs = *(const f32x4_t *)(sm + L::XC + (((kWaves - 1 - wv) * 4 + a) * 64 + lane) * 4);
                    ga = hf == 0 ? mine[a] : theirs;
                    da = hf == 0 ? theirs : mine[a];
                } else {
#pragma unroll
                    for (int kc = 0; kc < NPAD / 32; ++kc) {
                        float av[8], bv[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            av[j] = sC[(16 * a + l16) * BP + 32 * kc + 8 * g + j];
                            bv[j] = sB[s * BP + 32 * kc + 8 * g + j];
                        }
                        ga = mma8(av, bv, ga);
                    }
#pragma unroll
                    for (int kc = 0; kc < PPAD / 32; ++kc) {
                        float av[8], bv[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            av[j] = sY[(16 * a + l16) * XP + 32 * kc + 8 * g + j];
                            bv[j] = sX[s * XP + 32 * kc + 8 * g + j];
                        }
                        da = mma8(av, bv, da);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * a + 4 * g + i, tok_t = rtok(t);
                    const bool later = tok_t > tok_s, same = tok_t == tok_s;
                    const float ev = later ? __expf(rcs(t) - cs_s) : 0.f;
                    const float lv = later ? ev * kap_s : (same ? rgam(t) : 0.f);
                    P1s[a][i] = lv * ga[i];
                    P2s[a][i] = lv * da[i];
                    const float gd = ga[i] * da[i];
                    ce += ev * gd;
                    rw[i] = kap_s * ev * gd;
                    rd[i] = same ? gd : 0.f;
                }
            }
            if (hf == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v1 = row_sum16(rw[i]), v2 = row_sum16(rd[i]);
                    if (l16 == 0) {
                        sm[L::RW + w * 64 + 16 * a + 4 * g + i] = v1;
                        sm[L::RD + w * 64 + 16 * a + 4 * g + i] = v2;
                    }
                }
            }
        }
        ce = rows_sum4(ce);
        if (hf == 0 && g == 0) sm[L::CE + s] = ce;
    }
    // dX intra (this half's p tiles) and dB~ intra (this half's n tiles): rows s = 16 w + 4 g + i
    f32x4_t accX[PH], accB[NH];
#pragma unroll
    for (int q = 0; q < PH; ++q) {
        const int bq = hf * PH + q;
        accX[q] = zero4();
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            if (2 * kc + 1 < amin) continue;
            float av[8], bv[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                av[j] = P1s[2 * kc][j];
                av[j + 4] = P1s[2 * kc + 1][j];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) bv[j] = sY[tile_k(kc, g, j) * XP + 16 * bq + l16];
            accX[q] = mma8(av, bv, accX[q]);
        }
    }
#pragma unroll
    for (int ns = 0; ns < NH; ++ns) {
        const int nq = 2 * ns + hf;
        accB[ns] = zero4();
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            if (2 * kc + 1 < amin) continue;
            float av[8], bv[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                av[j] = P2s[2 * kc][j];
                av[j + 4] = P2s[2 * kc + 1][j];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) bv[j] = sC[tile_k(kc, g, j) * BP + 16 * nq + l16];
            accB[ns] = mma8(av, bv, accB[ns]);
        }
    }
    // ------------------------------------------------ t-oriented triangle: lane value [a][i]: t = 16 w + l16, s = 16 a + 4 g + i
    f32x4_t accC[NH], accY[PH];
    {
        f32x4_t P2t[4], P1t[4];
        const int t = 16 * w + l16;
        const float cs_t = rcs(t), gam_t = rgam(t);
        const int tok_t = rtok(t);
        const bool gate = p.z != nullptr;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            P2t[a] = P1t[a] = zero4();
            if (a > amax) continue;
            f32x4_t da = zero4(), ga = zero4();
#pragma unroll
            for (int kc = 0; kc < PPAD / 32; ++kc) {
                float av[8], bv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    av[j] = sX[(16 * a + l16) * XP + 32 * kc + 8 * g + j];
                    bv[j] = sY[t * XP + 32 * kc + 8 * g + j];
                }
                da = mma8(av, bv, da);
            }
            if (gate) {
#pragma unroll
                for (int kc = 0; kc < NPAD / 32; ++kc) {
                    float av[8], bv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        av[j] = sB[(16 * a + l16) * BP + 32 * kc + 8 * g + j];
                        bv[j] = sC[t * BP + 32 * kc + 8 * g + j];
                    }
                    ga = mma8(av, bv, ga);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * a + 4 * g + i, tok_s = rtok(s);
                const float lv = tok_t > tok_s ? __expf(cs_t - rcs(s)) * rkap(s) : (tok_t == tok_s ? gam_t : 0.f);
                P2t[a][i] = lv * da[i];
                P1t[a][i] = lv * ga[i];
            }
        }
#pragma unroll
        for (int ns = 0; ns < NH; ++ns) {
            const int nq = 2 * ns + hf;
            accC[ns] = zero4();
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                if (2 * kc > amax) continue;
                float av[8], bv[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    av[j] = P2t[2 * kc][j];
                    av[j + 4] = P2t[2 * kc + 1][j];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) bv[j] = sB[tile_k(kc, g, j) * BP + 16 * nq + l16];
                accC[ns] = mma8(av, bv, accC[ns]);
            }
        }
#pragma unroll
        for (int q = 0; q < PH; ++q) {
            const int bq = hf * PH + q;
            accY[q] = zero4();
            if (!gate) continue;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                if (2 * kc > amax) continue;
                float av[8], bv[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    av[j] = P1t[2 * kc][j];
                    av[j + 4] = P1t[2 * kc + 1][j];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) bv[j] = sX[tile_k(kc, g, j) * XP + 16 * bq + l16];
                accY[q] = mma8(av, bv, accY[q]);
            }
        }
    }
    // ------------------------------------------------ state terms, one slab of 32 state rows at a time
    f32x4_t accXi[PH], accZ[NH], accCi[NH], accYi[PH];
#pragma unroll
    for (int q = 0; q < PH; ++q) accXi[q] = accYi[q] = zero4();
    float hdot = 0.f;
    float gk[SQ];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
        // adjoint after the chunk (Gb), rows 32 ns ..
        __syncthreads();
#pragma unroll
        for (int q = 0; q < SQ; ++q) {
            const int e = tid + kThreads * q, row = e / PPAD, col = e - row * PPAD;
            const float v = slab_ok(ns, q) ? stg[PFA ? 2 * ns : 0][q] : 0.f;
            sS[row * XP + col] = v;
            gk[q] = v;
        }
        __syncthreads();
        if constexpr (!PFA) load_slab(stg[0], Hst, ns);
#pragma unroll
        for (int q = 0; q < PH; ++q) {
            const int bq = hf * PH + q;
            float av[8], bv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                av[j] = sB[(16 * w + l16) * BP + 32 * ns + 8 * g + j];
                bv[j] = sS[(8 * g + j) * XP + 16 * bq + l16];
            }
            accXi[q] = mma8(av, bv, accXi[q]);
        }
        accZ[ns] = zero4();
#pragma unroll
        for (int kc = 0; kc < PPAD / 32; ++kc) {
            float av[8], bv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                av[j] = sX[(16 * w + l16) * XP + 32 * kc + 8 * g + j];
                bv[j] = sS[(16 * hf + l16) * XP + 32 * kc + 8 * g + j];
            }
            accZ[ns] = mma8(av, bv, accZ[ns]);
        }
        // state before the chunk (H), same rows
        __syncthreads();
#pragma unroll
        for (int q = 0; q < SQ; ++q) {
            const int e = tid + kThreads * q, row = e / PPAD, col = e - row * PPAD;
            const float v = slab_ok(ns, q) ? stg[PFA ? 2 * ns + 1 : 0][q] : 0.f;
            sS[row * XP + col] = v;
            hdot += gk[q] * v;
        }
        __syncthreads();
        if constexpr (!PFA) {
            if (ns + 1 < NS) load_slab(stg[0], Gend, ns + 1);
        }
        accCi[ns] = zero4();
#pragma unroll
        for (int kc = 0; kc < PPAD / 32; ++kc) {
            float av[8], bv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                av[j] = sY[(16 * w + l16) * XP + 32 * kc + 8 * g + j];
                bv[j] = sS[(16 * hf + l16) * XP + 32 * kc + 8 * g + j];
            }
            accCi[ns] = mma8(av, bv, accCi[ns]);
        }
        if (p.z) {
#pragma unroll
            for (int q = 0; q < PH; ++q) {
                const int bq = hf * PH + q;
                float av[8], bv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    av[j] = sC[(16 * w + l16) * BP + 32 * ns + 8 * g + j];
                    bv[j] = sS[(8 * g + j) * XP + 16 * bq + l16];
                }
                accYi[q] = mma8(av, bv, accYi[q]);
            }
        }
    }
    // ------------------------------------------------ epilogue 1: dx, dz, row partials, angle terms
    const float Dh = p.D[h];
    const int64_t bth0 = (b * T + t0) * H + h;  // (b, t0, h); token k adds k H
    float dph[NH][4];
    {
        const bool gz = p.z && p.dz;
        const ET *zp = (const ET *)(p.z ? p.z : p.x);
        const float *dpx = p.dpx1 ? p.dpx1 : p.dt;
        ET zr[PH][4], yr[PH][4];
        float xf[PH][4];
        bool eo[PH][4];
#pragma unroll
        for (int q = 0; q < PH; ++q) {
            const int pc = 16 * (hf * PH + q) + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * w + 4 * g + i, k = rtok(s), r = s - k * R;
                eo[q][i] = k < Tv && pc < P;
                const int64_t o = (bth0 + (int64_t)k * H) * P * R + (int64_t)pc * R + r;
                zr[q][i] = ld_raw(zp, o, eo[q][i] && gz);
                yr[q][i] = ld_raw((const ET *)p.dy, o, eo[q][i] && gz);
                const bool okf = eo[q][i] && last && k == Tv - 1 && p.dpx1;
                const float f = ld_raw(dpx, (bh * P + pc) * R + r, okf);
                xf[q][i] = okf ? f : 0.f;
            }
        }
#pragma unroll
        for (int q = 0; q < PH; ++q) {
            const int pc = 16 * (hf * PH + q) + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * w + 4 * g + i, k = rtok(s), r = s - k * R;
                if (!eo[q][i]) continue;
                const int64_t o = (bth0 + (int64_t)k * H) * P * R + (int64_t)pc * R + r;
                const float v = accX[q][i] + rdec(s) * rkap(s) * accXi[q][i] + Dh * sY[s * XP + pc] + xf[q][i];
                if (p.dx) Io::st((ET *)p.dx + o, v);
                if (gz) {
                    const float yp = accY[q][i] + recs(s) * accYi[q][i] + Dh * sX[s * XP + pc];
                    const float zv = raw_f<Io>(zr[q][i], true), sg = sigmoid_f(zv);
                    Io::st((ET *)p.dz + o, raw_f<Io>(yr[q][i], true) * yp * sg * (1.f + zv * (1.f - sg)));
                }
            }
        }
    }
    {
        float ksum[4] = {0.f, 0.f, 0.f, 0.f}, asum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ns = 0; ns < NH; ++ns) {
            const int n = 16 * (2 * ns + hf) + l16;
            // component (odd) and pair (i2) of column n, and the pair's other column; with the
            // half-split pairing (N = NPAD of 64 or 128) the other column n +- N/2 is in this
            // lane's slot ns +- NH/2
            const bool odd = HS ? n >= N2 : (n & 1) != 0;
            const int i2 = HS ? (odd ? n - N2 : n) : n >> 1;
            const int nx = HS ? (odd ? n - N2 : n + N2) : n ^ 1;
            float thc = 1.f, ths = 0.f;
            if (last && p.dpB1 && n < N && i2 < NR) fast_sincos(p.thst[bh * N2 + i2], ths, thc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * w + 4 * g + i, k = rtok(row), r = row - k * R;
                const float z = rdec(row) * accZ[ns][i];
                float db = accB[ns][i] + rkap(row) * z;
                if (last && k == Tv - 1 && p.dpB1 && n < N) {
                    const float d0 = p.dpB1[(bh * N + pc0<HS, NPAD>(i2)) * R + r], d1 = p.dpB1[(bh * N + pc1<HS, NPAD>(i2)) * R + r];
                    db += odd ? (-ths * d0 + thc * d1) : (thc * d0 + ths * d1);
                }
                const float ci = recs(row) * accCi[ns][i];
                const float dc = accC[ns][i] + ci;
                const float bn = sB[row * BP + n], cn = sC[row * BP + n];
                ksum[i] += bn * z;
                asum[i] += cn * ci;
                // <d, J v> over the pair: component 0 pairs with -v1, component 1 with v0
                const float bo = sB[row * BP + nx], co = sC[row * BP + nx];
                float term = odd ? (db * bo + dc * co) : -(db * bo + dc * co);
                if constexpr (!HS) term += dpp_f<0xB1>(term);  // adjacent pairs: the other column is lane ^ 1
                dph[ns][i] = term;
                accB[ns][i] = db;
                accC[ns][i] = dc;
            }
        }
        if constexpr (HS) {
            // half-split pairs: the two columns' terms are in slots ns and ns + NH/2
#pragma unroll
            for (int ns = 0; ns < NH / 2; ++ns)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float t = dph[ns][i] + dph[ns + NH / 2][i];
                    dph[ns][i] = t;
                    dph[ns + NH / 2][i] = t;
                }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float kv = row_sum16(ksum[i]), av = row_sum16(asum[i]);
            if (l16 == 0) {
                sm[L::KS + hf * 64 + 16 * w + 4 * g + i] = kv;
                sm[L::AT + hf * 64 + 16 * w + 4 * g + i] = av;
            }
        }
    }
    const float hd = block_sum(hdot, sm + L::MS);  // (its barriers end every read of x, dy, B~, C~)
    const float dD = block_sum(dDp, sm + L::MS + 8);
    // ------------------------------------------------ epilogue 2: angle terms and dB~, dC~ to LDS
    float *dphi = sm + L::SX;  // [64][N2P], over the x and dy rows
#pragma unroll
    for (int ns = 0; ns < NH; ++ns) {
        const int n = 16 * (2 * ns + hf) + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * w + 4 * g + i;
            if constexpr (HS) {
                if (n < N2) dphi[row * N2P + n] = n < NR ? dph[ns][i] : 0.f;
            } else if (!(n & 1)) {
                dphi[row * N2P + (n >> 1)] = (n >> 1) < NR ? dph[ns][i] : 0.f;
            }
            sB[row * BP + n] = accB[ns][i];
            sC[row * BP + n] = accC[ns][i];
        }
    }
    __syncthreads();
    // ------------------------------------------------ per-token scalars (wave 0; lane = row, then token)
    if (tid < 64) {
        const int row = tid, k = tid;
        const bool rv = row / R < Tv && row < Qt * R;
        float dcs_r = 0.f, dk_r = 0.f, dgd_r = 0.f, bst = 0.f;
        if (rv) {
            const float kap = rkap(row);
            const float rw = sm[L::RW + row] + sm[L::RW + 64 + row] + sm[L::RW + 128 + row] + sm[L::RW + 192 + row];
            const float ks = sm[L::KS + row] + sm[L::KS + 64 + row];
            const float ce = sm[L::CE + row];
            dcs_r = rw + sm[L::AT + row] + sm[L::AT + 64 + row] - kap * (ce + ks);
            dk_r = ce + ks;
            dgd_r = sm[L::RD + row] + sm[L::RD + 64 + row] + sm[L::RD + 128 + row] + sm[L::RD + 192 + row];
            bst = kap * ks;
        }
        const float btot = wave_sum(bst);
        float dcs = 0.f, dk = 0.f, dgd = 0.f;
        if (R == 1) {
            // one row per token: the row of token k is lane k
            dcs = dcs_r;
            dk = dk_r;
            dgd = dgd_r;
        } else {
            for (int r = 0; r < R; ++r) {
                const int src = min(k * R + r, 63);
                const float a0 = __shfl(dcs_r, src, 64), a1 = __shfl(dk_r, src, 64), a2 = __shfl(dgd_r, src, 64);
                if (k * R + r < 64) {
                    dcs += a0;
                    dk += a1;
                    dgd += a2;
                }
            }
        }
        if (k >= Tv) dcs = dk = dgd = 0.f;
        // the chunk's last token: e^cs_end <Gb, H> and the state terms of every row
        if (k == Tv - 1) dcs += __expf(sm[L::TK + Tv - 1]) * hd + btot;
        // d log alpha_k = sum over the chunk's tokens >= k
        const float incl = wave_incl_scan(dcs);
        const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
        const float dla = tot - incl + dcs;
        if (k < Tv) {
            float *d = p.dsc + ((bh * T) + t0 + k) * 3;
            d[0] = dla;
            d[1] = dk + dgd;
            d[2] = dk;
        }
    }
    // ------------------------------------------------ angle gradients: per pair, sums over the ranks, reverse running sums
    {
        float *scr = sm + L::SS;  // [8][64]
        float dk8[8];
        float seg = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = 8 * wv + j;
            float v = 0.f;
            if (lane < N2P && k < Tv)
                for (int r = 0; r < R; ++r) v += dphi[(k * R + r) * N2P + lane];
            dk8[j] = v;
            seg += v;
        }
        if (lane < N2P) scr[wv * 64 + lane] = seg;
        __syncthreads();
        if (lane < N2P) {
            float run = 0.f;
            for (int ww = wv + 1; ww < kWaves; ++ww) run += scr[ww * 64 + lane];
            if (wv == 0 && lane < N2) p.tot[cidx * N2 + lane] = lane < NR ? run + seg : 0.f;
#pragma unroll
            for (int j = 7; j >= 0; --j) {
                const int k = 8 * wv + j;
                run += dk8[j];
                if (k < Tv && lane < NR && p.dtheta) p.dtheta[(bth0 + (int64_t)k * H) * NR + lane] = run;
            }
        }
        __syncthreads();
    }
    // ------------------------------------------------ un-rotation and norm backward of each B and C row
    {
        // raw B and C rows of this wave, loaded together
        using RP = RowPass<N2P>;
        constexpr int NM = RP::NM;
        const int pl = RP::pair();
        const int q0 = pc0<HS, NPAD>(pl), q1 = pc1<HS, NPAD>(pl);  // this lane's two columns
        ET rr[NM][2][2];
        bool ro[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int rho = RP::row(wv, m), k = rho / R, r = rho - k * R;
            ro[m] = k < Qt && k < Tv && pl < N2;
            const int64_t o = (bth0 + (int64_t)k * H) * N * R + r;
            rr[m][0][0] = ld_raw((const ET *)p.Bm, o + (int64_t)q0 * R, ro[m]);
            rr[m][0][1] = ld_raw((const ET *)p.Bm, o + (int64_t)q1 * R, ro[m]);
            rr[m][1][0] = ld_raw((const ET *)p.Cm, o + (int64_t)q0 * R, ro[m]);
            rr[m][1][1] = ld_raw((const ET *)p.Cm, o + (int64_t)q1 * R, ro[m]);
        }
        if constexpr (!L::KEEP) {
            AngleTile<N2P> ang;
            angle_load<N2P>(p, ang, b, h, t0, Tv);
            angle_scan<N2P>(ang, sm + L::PH, sm + L::RW);
        }
        // bias sums: per (side, rank, pair), over the chunk's tokens, of the un-rotated dB~ / dC~
        // (over the x and dy rows: [8][2][NPAD] per-wave gain sums, then either [8][2][NPAD]
        // per-wave bias sums or [2][R][NPAD] column bias sums; at most 32 NPAD floats).  When R divides 8 every row of a wave has rank
        // wv % R and the sums are taken in the row loop below; otherwise a pass over the columns.
        float *acc = sm + L::SX;
        const bool rdiv = (8 % R) == 0;
        if (!rdiv)
        for (int e = tid; e < 2 * R * (NPAD / 2); e += kThreads) {
            const int side = e / (R * (NPAD / 2)), rem = e - side * R * (NPAD / 2), r = rem / (NPAD / 2),
                      i = rem - r * (NPAD / 2);
            const float *rows = side == 0 ? sB : sC;
            float a0 = 0.f, a1 = 0.f;
            for (int k = 0; k < Tv; ++k) {
                float sn, cn;
                fast_sincos(sm[L::PH + k * N2P + i], sn, cn);
                const float e0 = rows[(k * R + r) * BP + pc0<HS, NPAD>(i)], e1 = rows[(k * R + r) * BP + pc1<HS, NPAD>(i)];
                a0 += cn * e0 + sn * e1;
                a1 += -sn * e0 + cn * e1;
            }
            acc[16 * NPAD + (side * R + r) * NPAD + pc0<HS, NPAD>(i)] = a0;
            acc[16 * NPAD + (side * R + r) * NPAD + pc1<HS, NPAD>(i)] = a1;
        }
        __syncthreads();
        const bool norm = (p.flags & kFlagNorm) != 0;
        float ga[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // this lane's gain sums (pair pl)
        float ba[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // this lane's bias sums (rank wv % R)
        const float invN = 1.f / (float)N;
        const float *phi = sm + L::PH;
        float gn[2][2];
        {
            const float *bnp = p.bnw ? p.bnw : p.dt, *cnp = p.cnw ? p.cnw : p.dt;
            const bool okb = pl < N2 && p.bnw, okc = pl < N2 && p.cnw;
            gn[0][0] = ld_raw(bnp, q0, okb);
            gn[0][1] = ld_raw(bnp, q1, okb);
            gn[1][0] = ld_raw(cnp, q0, okc);
            gn[1][1] = ld_raw(cnp, q1, okc);
            gn[0][0] = okb ? gn[0][0] : 1.f;
            gn[0][1] = okb ? gn[0][1] : 1.f;
            gn[1][0] = okc ? gn[1][0] : 1.f;
            gn[1][1] = okc ? gn[1][1] : 1.f;
        }
        const int lp = pl < N2P ? pl : 0;  // clamped pair for the LDS reads
        const int l0 = pc0<HS, NPAD>(lp), l1 = pc1<HS, NPAD>(lp);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int rho = RP::row(wv, m), k = rho / R;
            const bool rok = k < Qt && k < Tv;
            if (__ballot(rok) == 0) continue;  // neither row of the wave is in the chunk
            const bool lv = rok && pl < N2;
            float sn, cn;
            fast_sincos(phi[(rok ? k : 0) * N2P + lp], sn, cn);
#pragma unroll
            for (int side = 0; side < 2; ++side) {
                float *rows = side == 0 ? sB : sC;
                const float v0 = raw_f<Io>(rr[m][side][0], ro[m]), v1 = raw_f<Io>(rr[m][side][1], ro[m]);
                const float g0 = gn[side][0], g1 = gn[side][1];
                const float e0 = rows[rho * BP + l0], e1 = rows[rho * BP + l1];
                const float d0 = lv ? cn * e0 + sn * e1 : 0.f, d1 = lv ? -sn * e0 + cn * e1 : 0.f;
                float o0 = d0, o1 = d1;
                if (norm) {
                    const float rs = L::KEEP ? sm[L::RS + 64 * side + rho]
                                             : rsqrtf(RP::sum(v0 * v0 + v1 * v1) * invN + p.eps);
                    const float dot = RP::sum(d0 * g0 * v0 + d1 * g1 * v1);
                    const float f = dot * rs * rs * rs * invN;
                    o0 = d0 * g0 * rs - f * v0;
                    o1 = d1 * g1 * rs - f * v1;
                    ga[side][0] += d0 * v0 * rs;
                    ga[side][1] += d1 * v1 * rs;
                }
                ba[side][0] += d0;
                ba[side][1] += d1;
                if (lv) {
                    rows[rho * BP + q0] = o0;
                    rows[rho * BP + q1] = o1;
                }
            }
        }
        // both halves of the wave hold sums for the same pairs (ranks agree when R divides 8)
#pragma unroll
        for (int side = 0; side < 2; ++side)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                ga[side][j] += RP::other(ga[side][j]);
                ba[side][j] += RP::other(ba[side][j]);
            }
        if (RP::half() == 0 && pl < NPAD / 2)
#pragma unroll
            for (int side = 0; side < 2; ++side) {
                acc[(wv * 2 + side) * NPAD + q0] = ga[side][0];
                acc[(wv * 2 + side) * NPAD + q1] = ga[side][1];
                if (rdiv) {
                    acc[16 * NPAD + (wv * 2 + side) * NPAD + q0] = ba[side][0];
                    acc[16 * NPAD + (wv * 2 + side) * NPAD + q1] = ba[side][1];
                }
            }
    }
    __syncthreads();
    // dB and dC, in memory order (token, n, rank)
#pragma unroll
    for (int side = 0; side < 2; ++side) {
        ET *out = (ET *)(side == 0 ? p.dB : p.dC);
        if (!out) continue;
        const float *rows = side == 0 ? sB : sC;
        constexpr int E = 16 / Io::bytes;
        if (R == 1 && N % E == 0) {
            // single-rank rows: 16-byte stores of E consecutive elements (N a multiple of E
            // keeps every row start 16-byte aligned)
            const int ne = N / E;
            for (int e = tid; e < Tv * ne; e += kThreads) {
                const int k = e / ne, n = E * (e - k * ne);
                const float *src = rows + k * BP + n;
                u32x4_t v;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (Io::bytes == 2)
                        v[j] = (uint32_t)f2bf(src[2 * j]) | ((uint32_t)f2bf(src[2 * j + 1]) << 16);
                    else
                        v[j] = __float_as_uint(src[j]);
                }
                *reinterpret_cast<u32x4_t *>(out + (bth0 + (int64_t)k * H) * N + n) = v;
            }
        } else {
            for (int e = tid; e < Tv * N * R; e += kThreads) {
                const int k = e / (N * R), rem = e - k * N * R, n = rem / R, r = rem - n * R;
                Io::st(out + (bth0 + (int64_t)k * H) * N * R + rem, rows[(k * R + r) * BP + n]);
            }
        }
    }
    const float *acc = sm + L::SX;
    float *part = p.part + cidx * (int64_t)p.pw;
    for (int e = tid; e < 2 * N; e += kThreads) {
        const int side = e / N, n = e - side * N;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) v += acc[(ww * 2 + side) * NPAD + n];
        part[3 + e] = v;
    }
    for (int e = tid; e < 2 * R * N; e += kThreads) {
        const int side = e / (R * N), rn = e - side * R * N, r = rn / N, n = rn - r * N;
        float v = 0.f;
        if ((8 % R) == 0) {
            for (int ww = r; ww < kWaves; ww += R) v += acc[16 * NPAD + (ww * 2 + side) * NPAD + n];
        } else {
            v = acc[16 * NPAD + (side * R + r) * NPAD + n];
        }
        part[3 + 2 * N + e] = v;
    }
    if (tid == 0) part[1] = dD;
}

// ---------------------------------------------------------------- angle gradient suffix sums
// tot[c] <- final-angle gradient + sum of tot over the chunks after c.
__global__ __launch_bounds__(kThreads) void bwd_angle_suffix_kernel(BwdParams p) {
    __shared__ float scr[kWaves][64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int N2 = p.N / 2, NR = p.nr, nck = p.nck;
    const int per = (nck + kWaves - 1) / kWaves;
    const int c0 = wv * per, c1 = min(nck, c0 + per);
    float *tot = p.tot + bh * nck * (int64_t)N2;
    float s = 0.f;
    if (lane < NR)
        for (int c = c0; c < c1; ++c) s += tot[(int64_t)c * N2 + lane];
    scr[wv][lane] = s;
    __syncthreads();
    if (lane >= NR) return;
    float run = p.dang1 ? p.dang1[bh * NR + lane] : 0.f;
    for (int ww = wv + 1; ww < kWaves; ++ww) run += scr[ww][lane];
    for (int c = c1 - 1; c >= c0; --c) {
        const float v = tot[(int64_t)c * N2 + lane];
        tot[(int64_t)c * N2 + lane] = run;
        run += v;
    }
}

// ---------------------------------------------------------------- initial state
// h_init, prev_B, prev_x enter as H_0 = Rot(-Theta_init)(h_init + eta_{-1} prev_B prev_x^T);
// G0w holds the adjoint of h_init + eta_{-1} prev_B prev_x^T (global frame).
// The initial angle's gradient comes from rotating the whole frame by the same angle,
// which changes only the states at both ends (the loss sees the final state):
//   d Theta_init = d Theta_final + <dh_final, J h_final> + <dprevB_final, J prevB_final>
//                  - <dh_init, J h_init> - <dprevB_init, J prevB_init>      (per pair)
// with <a, J v> = -a_0 v_1 + a_1 v_0; exact zero when no state enters or leaves.
template <class Io>
__global__ __launch_bounds__(256) void bwd_init_kernel(BwdParams p) {
    using ET = typename Io::T;
    __shared__ float red[4];
    __shared__ float sang[4][64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H;
    const int h = (int)(bh - b * p.H);
    const int N = p.N, P = p.P, R = p.R, N2 = N / 2, NR = p.nr, nck = p.nck;
    M3_DCHECK(p, bh < p.B * p.H);
    const int64_t T = p.T;
    const float *G0 = p.G0w + bh * N * (int64_t)P;
    if (p.dh0)
        for (int e = tid; e < N * P; e += 256) p.dh0[bh * N * (int64_t)P + e] = G0[e];
    const float eta = eta_at(p, b, h, -1);
    float de = 0.f;
    for (int e = tid; e < N * R; e += 256) {
        const int n = e / R, r = e - n * R;
        float s = 0.f;
        if (p.px0)
            for (int pc = 0; pc < P; ++pc) s += G0[(int64_t)n * P + pc] * p.px0[(bh * P + pc) * R + r];
        if (p.dpB0) p.dpB0[(bh * N + n) * R + r] = eta * s;
        if (p.pB0) de += p.pB0[(bh * N + n) * R + r] * s;
    }
    for (int e = tid; e < P * R; e += 256) {
        const int pc = e / R, r = e - pc * R;
        float s = 0.f;
        if (p.pB0)
            for (int n = 0; n < N; ++n) s += G0[(int64_t)n * P + pc] * p.pB0[(bh * N + n) * R + r];
        if (p.dpx0) p.dpx0[(bh * P + pc) * R + r] = eta * s;
    }
    de = wave_sum(de);
    if (lane == 0) red[wv] = de;
    // initial angle: wave wv sums its share of the columns per pair (lane = pair)
    float a = 0.f;
    if (lane < NR) {
        const int i = lane, n0 = pn0(p, i), n1 = pn1(p, i);
        const float *Gl = p.Ust + (bh * nck + nck - 1) * N * (int64_t)P;  // adjoint after the last chunk
        const float *Hf = p.hfin + bh * N * (int64_t)P;                     // state after it, same frame
        for (int pc = wv; pc < P; pc += 4) {
            const int64_t o0 = (int64_t)n0 * P + pc, o1 = (int64_t)n1 * P + pc;
            a += -Gl[o0] * Hf[o1] + Gl[o1] * Hf[o0];
            if (p.h0) a -= -G0[o0] * p.h0[bh * N * (int64_t)P + o1] + G0[o1] * p.h0[bh * N * (int64_t)P + o0];
        }
        for (int r = wv; r < R; r += 4) {
            if (p.pB0) {
                // dprev_B_init = eta G0 prev_x (as above)
                float d0 = 0.f, d1 = 0.f;
                if (p.px0)
                    for (int pc = 0; pc < P; ++pc) {
                        const float xv = p.px0[(bh * P + pc) * R + r];
                        d0 += G0[(int64_t)n0 * P + pc] * xv;
                        d1 += G0[(int64_t)n1 * P + pc] * xv;
                    }
                d0 *= eta;
                d1 *= eta;
                a -= -d0 * p.pB0[(bh * N + n1) * R + r] + d1 * p.pB0[(bh * N + n0) * R + r];
            }
        }
    }
    // prev_B of the final state: the normalised, biased B of the last token rotated by the
    // final angle; <dprevB, J Rot(Theta) b> = <Rot(-Theta) dprevB, J b>
    if (p.dpB1)
        for (int r = wv; r < R; r += 4) {
            const int64_t bth = (b * T + T - 1) * p.H + h;
            const ET *raw = (const ET *)p.Bm + bth * N * R + r;
            const bool norm = (p.flags & kFlagNorm) != 0;
            float v0 = 0.f, v1 = 0.f;
            const int n0 = pn0(p, lane), n1 = pn1(p, lane);  // lane = pair
            if (lane < N2) {
                v0 = Io::ld(raw + (int64_t)n0 * R);
                v1 = Io::ld(raw + (int64_t)n1 * R);
            }
            const float rs = norm ? rsqrtf(wave_sum(v0 * v0 + v1 * v1) / (float)N + p.eps) : 1.f;
            if (lane < NR) {
                const int i = lane;
                float b0 = norm ? v0 * rs * (p.bnw ? p.bnw[n0] : 1.f) : v0;
                float b1 = norm ? v1 * rs * (p.bnw ? p.bnw[n1] : 1.f) : v1;
                if (p.bbias) {
                    b0 += p.bbias[((int64_t)h * R + r) * N + n0];
                    b1 += p.bbias[((int64_t)h * R + r) * N + n1];
                }
                const float th = (float)wrap_2pi((double)p.thst[bh * N2 + i] + (double)p.phic[(bh * nck + nck - 1) * N2 + i]);
                float sn, cn;
                fast_sincos(th, sn, cn);
                const float e0 = p.dpB1[(bh * N + n0) * R + r], e1 = p.dpB1[(bh * N + n1) * R + r];
                const float f0 = cn * e0 + sn * e1, f1 = -sn * e0 + cn * e1;
                a += -f0 * b1 + f1 * b0;
            }
        }
    sang[wv][lane] = a;
    __syncthreads();
    if (tid == 0) p.deta0[bh] = red[0] + red[1] + red[2] + red[3];
    if (tid < NR && p.dang0)
        p.dang0[bh * NR + tid] = (p.dang1 ? p.dang1[bh * NR + tid] : 0.f) + sang[0][tid] + sang[1][tid] +
                                 sang[2][tid] + sang[3][tid];
}

// ---------------------------------------------------------------- per-token gradients
// d dt, d lambda, d A from the chunk kernel's per-token sums; angle gradients completed
// with the later chunks' sums; per-chunk records of the A and dt-bias gradients.
__global__ __launch_bounds__(256) void bwd_token_kernel(BwdParams p) {
    __shared__ float red[4][2];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nck = p.nck, NR = p.nr, N2 = p.N / 2;
    const int64_t bh = blockIdx.x / nck;
    const int c = (int)(blockIdx.x - bh * nck);
    const int64_t b = bh / p.H;
    const int h = (int)(bh - b * p.H);
    const int Qt = kRows / p.R;
    M3_DCHECK(p, bh < p.B * p.H && c < nck && (int64_t)c * Qt < p.T);
    const int64_t T = p.T, H = p.H, t0 = (int64_t)c * Qt;
    const int Tv = (int)min((int64_t)Qt, T - t0);
    const int64_t cidx = bh * nck + c;
    if (p.dtheta) {
        if ((NR & 3) == 0 && (N2 & 3) == 0) {
            // 16-byte read-modify-write of each token's angle gradients (rows of NR floats;
            // the row starts and the per-chunk totals are 16-byte aligned)
            const int nv = NR / 4;
            for (int e = tid; e < Tv * nv; e += 256) {
                const int k = e / nv, i = 4 * (e - k * nv);
                f32x4_t *d = (f32x4_t *)(p.dtheta + ((b * T + t0 + k) * H + h) * (int64_t)NR + i);
                *d += *(const f32x4_t *)(p.tot + cidx * N2 + i);
            }
        } else {
            for (int e = tid; e < Tv * NR; e += 256) {
                const int k = e / NR, i = e - k * NR;
                p.dtheta[((b * T + t0 + k) * H + h) * (int64_t)NR + i] += p.tot[cidx * N2 + i];
            }
        }
    }
    float aA = 0.f, aB = 0.f;
    if (tid < Tv) {
        const int64_t t = t0 + tid, bth = (b * T + t) * H + h;
        const float *d = p.dsc + (bh * T + t) * 3;
        // (deta0 is NULL when no initial state enters: its eta weight has no gradient)
        const float dprev = t == 0 ? (p.deta0 ? p.deta0[bh] : 0.f) : p.dsc[(bh * T + t - 1) * 3 + 2];
        float dt, lam, dsp, dsg;
        act_scalars(p, bth, h, dt, lam, dsp, dsg);
        const float Av = (p.flags & kFlagAPerToken) ? p.A[bth] : p.A[h];
        float ddt = d[0] * Av + d[1] * lam + dprev * (1.f - lam);
        float dlm = (d[1] - dprev) * dt;
        const float dAv = d[0] * dt;
        ddt *= dsp;
        dlm *= dsg;
        if (p.ddt) p.ddt[bth] = ddt;
        if (p.dlam) p.dlam[bth] = dlm;
        if (p.flags & kFlagAPerToken) {
            if (p.dAt) p.dAt[bth] = dAv;
        } else {
            aA = dAv;
        }
        if (p.flags & kFlagDtSoftplus) aB = ddt;
    }
    aA = wave_sum(aA);
    aB = wave_sum(aB);
    if (lane == 0) {
        red[wv][0] = aA;
        red[wv][1] = aB;
    }
    __syncthreads();
    if (tid == 0) {
        float *part = p.part + cidx * (int64_t)p.pw;
        part[0] = red[0][0] + red[1][0] + red[2][0] + red[3][0];
        part[2] = red[0][1] + red[1][1] + red[2][1] + red[3][1];
    }
}

// Parameter gradients: one workgroup per parameter element sums its per-(sequence, chunk)
// records in a fixed order.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p) {
    __shared__ float s_red[256];
    const int H = p.H, N = p.N, R = p.R;
    const int64_t Bn = p.B;
    const int e = blockIdx.x, tid = threadIdx.x;
    const int nH = 3 * H, nG = 2 * N;
    const int nck = p.nck;
    float *dst = nullptr;
    float v = 0.f;
    if (e < nH) {
        const int which = e / H, h = e - which * H;  // 0: A, 1: D, 2: dt bias
        dst = which == 0 ? p.dA : (which == 1 ? p.dD : p.ddtb);
        if (dst) dst += h;
        for (int64_t k = tid; k < Bn * nck; k += 256) {
            const int64_t b = k / nck;
            v += p.part[((b * H + h) * nck + (k - b * nck)) * (int64_t)p.pw + which];
        }
    } else if (e < nH + nG) {
        const int k2 = e - nH, side = k2 / N, n = k2 - side * N;
        dst = side == 0 ? p.dbnw : p.dcnw;
        if (dst) dst += n;
        for (int64_t s = tid; s < Bn * H * nck; s += 256) v += p.part[s * p.pw + 3 + side * N + n];
    } else {
        const int k2 = e - nH - nG, side = k2 / (H * R * N), rem = k2 - side * (H * R * N);
        const int h = rem / (R * N), rn = rem - h * (R * N);
        dst = side == 0 ? p.dbb : p.dcb;
        if (dst) dst += rem;
        for (int64_t k = tid; k < Bn * nck; k += 256) {
            const int64_t b = k / nck;
            v += p.part[((b * H + h) * nck + (k - b * nck)) * (int64_t)p.pw + 3 + 2 * N + side * R * N + rn];
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

namespace {

template <int NPAD, int PPAD, bool GRAD, bool VEC = false>
constexpr size_t chunk_lds() { return sizeof(float) * CL<NPAD, PPAD, GRAD, !GRAD && state_split<NPAD, PPAD, VEC>()>::TOTAL; }

template <class Io, int NPAD, int PPAD, bool VEC>
hipError_t launch_chunks_v(const BwdParams &p, hipStream_t st) {
    const size_t lds = chunk_lds<NPAD, PPAD, false, VEC>(), ldg = chunk_lds<NPAD, PPAD, true>();
    const dim3 grid((unsigned)(p.B * p.H * p.nck)), blk(kThreads);
    // the half-split pairing in the chunk kernels needs N = NPAD of 64 or 128
    if (p.hs && (NPAD < 64 || p.N != NPAD)) return hipErrorInvalidValue;
    constexpr bool HSOK = NPAD >= 64;  // (no half-split variants below 64)
    const bool hs = HSOK && p.hs;
    const void *sk = hs ? (const void *)bwd_chunk_state_kernel<Io, NPAD, PPAD, VEC, HSOK>
                        : (const void *)bwd_chunk_state_kernel<Io, NPAD, PPAD, VEC, false>;
    const void *gk = hs ? (const void *)bwd_chunk_grad_kernel<Io, NPAD, PPAD, HSOK>
                        : (const void *)bwd_chunk_grad_kernel<Io, NPAD, PPAD, false>;
    hipError_t e;
    if ((e = hipFuncSetAttribute(sk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute(gk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldg)) != hipSuccess) return e;
    if (hs) hipLaunchKernelGGL((bwd_chunk_state_kernel<Io, NPAD, PPAD, VEC, HSOK>), grid, blk, lds, st, p);
    else hipLaunchKernelGGL((bwd_chunk_state_kernel<Io, NPAD, PPAD, VEC, false>), grid, blk, lds, st, p);
    const int64_t ne = p.B * p.H * (p.N / 2) * (int64_t)p.P;
    hipLaunchKernelGGL(bwd_state_pass_kernel, dim3((unsigned)((ne + 255) / 256), 2), dim3(256), 0, st, p);
    if (hs) hipLaunchKernelGGL((bwd_chunk_grad_kernel<Io, NPAD, PPAD, HSOK>), grid, blk, ldg, st, p);
    else hipLaunchKernelGGL((bwd_chunk_grad_kernel<Io, NPAD, PPAD, false>), grid, blk, ldg, st, p);
    return hipGetLastError();
}

template <class Io, int NPAD, int PPAD>
hipError_t launch_chunks(const BwdParams &p, hipStream_t st) {
    return p.vec ? launch_chunks_v<Io, NPAD, PPAD, true>(p, st) : launch_chunks_v<Io, NPAD, PPAD, false>(p, st);
}

template <class Io, int NPAD>
hipError_t launch_np(const BwdParams &p, hipStream_t st) {
    if (p.P <= 32) return launch_chunks<Io, NPAD, 32>(p, st);
    if (p.P <= 64) return launch_chunks<Io, NPAD, 64>(p, st);
    return launch_chunks<Io, NPAD, 128>(p, st);
}

template <class Io>
hipError_t launch_io(const BwdParams &p, hipStream_t st) {
    if (p.N <= 32) return launch_np<Io, 32>(p, st);
    if (p.N <= 64) return launch_np<Io, 64>(p, st);
    return launch_np<Io, 128>(p, st);
}

}  // namespace

hipError_t launch_bwd(bool bf16, const BwdParams &p, hipStream_t st) {
    if (p.T == 0) {
        const int64_t nbh = p.B * p.H;
        int64_t m = nbh * p.N * p.P;
        const int64_t others[] = {nbh * p.N * p.R, nbh * p.P * p.R, (int64_t)p.H * p.R * p.N, p.N, p.H};
        for (int64_t o : others) m = o > m ? o : m;
        if (m > 0) hipLaunchKernelGGL(bwd_empty_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, p);
        return hipGetLastError();
    }
    hipError_t e = bf16 ? launch_io<IoBF16>(p, st) : launch_io<IoF32>(p, st);
    if (e != hipSuccess) return e;
    const unsigned nbh = (unsigned)(p.B * p.H);
    hipLaunchKernelGGL(bwd_angle_suffix_kernel, dim3(nbh), dim3(kThreads), 0, st, p);
    // The initial-state kernel has work only when an initial state enters (its eta-weighted
    // prev_B prev_x^T term feeds d dt and d lambda of the first token) or a gradient of the
    // initial state is requested; otherwise the token kernel takes that term as zero.
    BwdParams pt = p;
    if (p.dh0 || p.dpB0 || p.dpx0 || p.dang0 || (p.pB0 && p.px0)) {
        if (bf16) hipLaunchKernelGGL(bwd_init_kernel<IoBF16>, dim3(nbh), dim3(256), 0, st, p);
        else hipLaunchKernelGGL(bwd_init_kernel<IoF32>, dim3(nbh), dim3(256), 0, st, p);
    } else {
        pt.deta0 = nullptr;
    }
    hipLaunchKernelGGL(bwd_token_kernel, dim3((unsigned)(nbh * p.nck)), dim3(256), 0, st, pt);
    const int total = 3 * p.H + 2 * p.N + 2 * p.H * p.R * p.N;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)total), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace m3
