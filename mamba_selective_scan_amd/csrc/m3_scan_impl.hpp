// m3_scan_impl.hpp -- the chunked Mamba-3 scan on gfx950 (kernel templates).
//
// Method.  Chunkwise SSD (torchmamba README, "Math notes", M2: an intra-chunk
// quadratic part plus a factored state carry between chunks) applied to the
// Mamba-3 trapezoid in its single-scan form (dotLLM PR #136, comment
// "Mamba-3 streaming decode": per-token scale gamma_t + eta_t with the
// one-token lookahead eta_t = dt_{t+1}(1 - lambda_{t+1}), which crosses block
// edges).  With the shifted state h'_t = h_t + eta_t B~_t x_t^T:
//     h'_t = alpha_t h'_{t-1} + (gamma_t + eta_t) B~_t x_t^T
//     y_t  = C~_t^T h'_t - eta_t (C~_t . B~_t) x_t + D x_t
// so inside a block the mask is
//     L[t, s] = exp(cs_t - cs_s) * (s < t ? scale_s : s == t ? gamma_t : 0)
// with cs the running sum of dt*A inside the block.  Rotations use
// block-local angles (running sum of theta from the block start); a carried
// state lives in the frame of the block it enters:
//     H_next = Rot(-Phi_end) (exp(cs_end) H + S),   S = sum_s exp(cs_end - cs_s) scale_s B~_s x_s^T.
//
// Work split.  A block is 64 rows ((token, rank) pairs, rank fastest).  The
// blocks of one (batch, head) sequence are cut into segments, and the head
// dimension P into column groups of at most 64; a workgroup walks the blocks
// of one segment in order for one column group, carrying the state in
// registers:
//   seg_state_kernel : per segment, the state it contributes starting from zero
//                      (to the workspace; not run for the last segment).
//   seg_output_kernel: per segment, the incoming state (initial state folded
//                      through the earlier segments' contributions), then for
//                      each block the outputs and the state update.
// No workgroup waits for another: the output kernel reads only what the state
// kernel, launched before it on the same stream, wrote.
//
// Matrix cores.  Wave w owns rows 16w..16w+15 of a block.
//   G^T tiles  = B~[s rows] C~[t rows]^T    (A: B~ from LDS, B: C~ in registers)
//   Y_intra   += (G o L) X                  (the G^T result fragments are the A operand)
//   Y_inter    = C~ H                       (B: H^T from LDS)
//   S          = (w B~)^T X                 (A: (w B~)^T, B: X^T, both from LDS)
// The state fragments hold S[n = 4g + i][p = l16] per 16x16 tile, so the two
// components of a rotation pair sit in one lane.
// bf16 I/O: every inexact operand is split into hi + lo bf16 and multiplied
// as hi*hi + hi*lo + lo*hi (x itself is exact); fp32 I/O uses the fp32 MFMA.
#pragma once
#include <type_traits>

#include "m3_device.hpp"
#include "m3_internal.hpp"

namespace m3 {

// LDS-only workgroup barrier (global memory needs no ordering between the waves here)
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Thread index inside the workgroup of 256 (4 waves), as the helpers below use it: the mask
// states the range to the compiler (the output kernel's register count fell from 241 to 232
// and its time by 4.7% at N = P = 64 when the helpers indexed by this instead of threadIdx.x).
__device__ __forceinline__ int ltid() { return (int)(threadIdx.x & 255u); }

// The 16-row tile of a block that this wave owns (wave-uniform: held in a scalar register, so
// that loops and branches on it are scalar).
__device__ __forceinline__ int row_tile() { return __builtin_amdgcn_readfirstlane(ltid() >> 6); }

// Load paths (the MODE of a kernel variant):
//   kModeGen : any rank, any even N, any P; element loads.
//   kModeVec : rank 1 with N and P multiples of 8; 16-byte loads straight into the
//              operand registers, angle running sums in registers.
//   kModeMimo: bf16, rank 2, 4 or 8 with N and P multiples of 8; 16-byte loads of the
//              (n, rank) / (p, rank) interleaved rows, regrouped per rank through LDS.
constexpr int kModeGen = 0, kModeVec = 1, kModeMimo = 2;

// SWZ_: XOR-swizzled X^T plane on the rank-1 16-byte path (see xt_off).
// PJ_: the variant that reads the MIMO projections (mimo_x, mimo_z, mimo_o) when given; the
// kernels without it never test for them (element and interleaved-rank paths only).
// HS_: the half-split rotation pairing (pair i = components (i, i + N/2)) natively, on the rank-1
// 16-byte path with N = NP (64 or 128): component kk*32 + 8g + j of a lane pairs with the same
// slot of step kk + KS/2 in the same lane, and state tile m (rows below N/2) with tile m + HSM.
template <class Io, int NP_, int PP_, int MODE_, bool SWZ_ = true, bool PJ_ = false, bool HS_ = false>
struct SegCfg {
    using ET = typename Io::T;
    static constexpr bool BF = std::is_same<Io, IoBF16>::value;
    static constexpr bool VEC = MODE_ == kModeVec;
    static constexpr bool MV = MODE_ == kModeMimo;
    static constexpr bool PJ = PJ_;
    static_assert(!PJ || !VEC, "the rank-1 16-byte path takes no projections");
    static constexpr bool HS = HS_;
    static_assert(!HS || (VEC && NP_ >= 64), "native half-split pairing: rank-1 16-byte path, N >= 64");
    static constexpr bool XSWZ = SWZ_ && VEC;
    static_assert(!MV || BF, "the interleaved-rank load path is bf16 only");
    static constexpr bool PACKED = (VEC || MV) && BF;  // raw B/C held as packed bf16 words
    static constexpr int NP = NP_, PP = PP_;
    static constexpr int ROWS = kBlockRows;
    static constexpr int KS = NP / 32;  // 32-wide k steps over n
    static constexpr int PT = PP / 16;  // p tiles
    static constexpr int NT = NP / 16;  // n tiles
    static constexpr int TPW = (PT * NT + 3) / 4;  // state tiles per wave
    static constexpr int HSM = (NT / 2) * PT / 4;  // half-split: partner of state tile m < HSM
    static constexpr int ES = BF ? 2 : 4;          // bytes per operand element per plane
    static constexpr int NPL = BF ? 2 : 1;         // planes: (hi, lo) or (fp32)
    // bf16 I/O: B~, C~ and H are single fp16 operands (power-of-two scaled); (w B~)^T, G o L
    // and X stay bf16 hi/lo (X exact).  The interleaved-rank path stages raw B and C in two
    // planes of the B~ area, so that area keeps two planes there.
    static constexpr bool F16 = BF;
    static constexpr int NPL_BT = F16 ? (MV ? 2 : 1) : NPL;
    static constexpr int NPL_HT = F16 ? 1 : NPL;
    // Column-owned outputs (rank-1 bf16 path with 64 columns): wave w computes Y^T for columns
    // 16w .. 16w + 15 and every row of the block, from the state columns it holds and from
    // G o L tiles computed once (spread evenly over the waves) and shared through LDS.
    static constexpr bool COL = VEC && F16 && PP == 64;
    static constexpr int PADE = BF ? 8 : 4;        // 16 bytes of padding per row
    static constexpr int OPP = NP + PADE;          // pitch of [row][n] and [p][n]
    static constexpr int RPP = ROWS + PADE;        // pitch of [p][row] and [n][row]
    static constexpr int PHP = NP / 2;             // pitch of the angle table [token][pair]
    static constexpr int XW = BF ? 8 : 4;          // io elements per 16-byte vector
    // per-thread raw counts
    static constexpr int XN = VEC ? (ROWS * PP / XW / 256) * 4 : ROWS * PP / 256;  // x words / elements
    // tokens per block: 64 for ranks 1 and 3..7 of the general path; at most 32 with MV (rank >= 2)
    static constexpr int TOKS = MV ? ROWS / 2 : ROWS;
    static constexpr int TN = VEC ? 4 * KS : TOKS * (NP / 2) / 256;               // theta floats
    static constexpr int BWV = BF ? 4 : 8;  // words per 8 B/C elements when VEC
    // MV: 16-byte vectors per thread for a block's B (or C) and x
    static constexpr int NBV = (ROWS * NP / 8 + 255) / 256;
    static constexpr int NXV = (ROWS * PP / 8 + 255) / 256;

    static constexpr size_t al(size_t v) { return (v + 15) / 16 * 16; }
    static constexpr size_t BT_PLANE = (size_t)ROWS * OPP;  // elements per plane
    static constexpr size_t WB_PLANE = (size_t)NP * RPP;
    static constexpr size_t HT_PLANE = (size_t)PP * OPP;
    static constexpr size_t L_BT = al(BT_PLANE * ES * NPL_BT);
    static constexpr size_t L_WB = al(WB_PLANE * ES * NPL);
    static constexpr size_t L_XT = al((size_t)PP * RPP * ES);
    static constexpr size_t L_HT = COL ? 0 : al(HT_PLANE * ES * NPL_HT);
    // y staging: the per-wave rows in the io type; fp32 in the projection variant, whose rank
    // contraction (mimo_o) sums fp32 per-rank terms there
    static constexpr size_t L_Y = COL ? 0 : al((size_t)ROWS * PP * (PJ ? 4 : sizeof(ET)));
    // COL: the C~ plane [row][n] (fp16) and the G o L planes [t][s] (bf16 hi, lo)
    static constexpr size_t L_CT = COL ? al(BT_PLANE * 2) : 0;
    static constexpr size_t GL_PLANE = (size_t)ROWS * RPP;
    static constexpr size_t L_GL = COL ? al(GL_PLANE * 2 * 2) : 0;
    // angles: the general path keeps a table [token][pair]; the SISO path only tile totals [4][pair]
    static constexpr size_t L_PHI = al(VEC ? (size_t)4 * (NP / 2) * 4 : (size_t)TOKS * PHP * 4);
    // scalars: per pair (cos, sin) of the block angle total [NP/2][2] (padded pairs (1, 0));
    // cs, scale, gamma, w, exp(cs), u (factored mask) [ROWS]; inverse row scales of B~ and
    // C~ [2][ROWS]; scan scratch [256 + 8]; per pair the block angle total; per wave the
    // largest |H|; per pair (double): running angle base
    static constexpr size_t L_SC0 = al((NP + 8 * ROWS + 264 + NP / 2 + 4) * 4);
    static constexpr size_t L_SC = L_SC0 + (size_t)(NP / 2) * 8;
    // MV state kernel: raw B regrouped per rank, [row][n] (the output kernel uses the B~ planes)
    static constexpr size_t L_RAW = MV ? al((size_t)ROWS * OPP * 2) : 0;
    // rank-1 path: norm gains and this head's biases for B and C, [4][NP] (1 and 0 when absent)
    static constexpr size_t L_AFF = VEC ? al((size_t)4 * NP * 4) : 0;
    static constexpr size_t STATE_BYTES = L_WB + L_XT + L_PHI + L_SC + L_RAW + L_AFF;
    static constexpr size_t OUTPUT_BYTES = L_BT + L_CT + L_GL + L_WB + L_XT + L_HT + L_Y + L_PHI + L_SC + L_AFF;
};

// Raw inputs of one block, prefetched into registers.  With VEC the words are
// the unconverted 16-byte loads; otherwise they are float bits.
template <class Cfg, bool WANT_C>
struct RawBlock {
    static constexpr int BW = Cfg::PACKED ? 4 : 8;  // words per 8 values
    static constexpr int NB = Cfg::MV ? Cfg::NBV : Cfg::KS;
    uint32_t b[NB][BW];  // MV: 16-byte vectors in memory order
    uint32_t c[WANT_C ? NB : 1][BW];
    uint32_t x[Cfg::MV ? Cfg::NXV * 4 : Cfg::XN];
    float th[Cfg::TN];
    float dt, lam, dtn, lamn;  // raw dt, lambda of the lane's token and the next one (wave 0)
    float av;                  // per-token decay rate of the lane's token (wave 0, kFlagAPerToken)
};

// Gate input z of one block, prefetched into registers with the same element mapping as x.
template <class Cfg>
struct RawZ {
    uint32_t w[Cfg::MV ? Cfg::NXV * 4 : Cfg::XN];
};

// Offset of (col, row) in the (w B~)^T plane [n][row] (pitch RPP), the row index
// XOR-swizzled by bits 3..5 of n.  The prologue writes one row into n, n + 8, ...
// at once; the swizzle spreads those writes over the LDS banks, and every aligned
// group of 8 rows stays contiguous for the 16-byte operand reads.
template <class Cfg>
__device__ __forceinline__ int tr_off(int col, int row) {
    return col * Cfg::RPP + (row ^ (((col >> 3) & 7) << 3));
}
// Offset of (row, col) in the y staging plane [row][PP] (rank-1 and general paths):
// columns XOR-swizzled in groups of 16 by bits 2.. of the row, so that the four
// 4-row groups written by one instruction use different banks.
// Offset of (p, row) in the X^T plane [p][row] (pitch RPP).  With XSWZ (rank-1 16-byte path)
// the row index is XOR-swizzled by bits 3..5 of p, as in the (w B~)^T plane: the staging
// writes one token's 8 consecutive p at once from 8 lanes per token, which without the
// swizzle all fall into one LDS bank; aligned groups of 8 (and 4) rows stay contiguous for
// the operand reads.  The gated output kernel keeps the plain layout (the swizzled addresses
// cost it more register spills than the conflicts they remove: 66 -> 74 us).
template <class Cfg>
__device__ __forceinline__ int xt_off(int col, int row) {
    if constexpr (Cfg::XSWZ) return col * Cfg::RPP + (row ^ (((col >> 3) & 7) << 3));
    else return col * Cfg::RPP + row;
}
template <class Cfg>
__device__ __forceinline__ int ys_off(int row, int col) {
    return row * Cfg::PP + (col ^ (((row >> 2) & (Cfg::PP / 16 - 1)) << 4));
}

// First of the four rotation pairs of angle group q (0 .. KS-1) of lane group g: the pairs of the
// components kk*32 + 8g .. + 7 of k step kk = q (adjacent pairing), or, half-split, the
// components of k step q / 2 (which pair with step q / 2 + KS / 2), half q % 2 of them.
template <class Cfg>
__device__ __forceinline__ int pair_off(int q, int g) {
    if constexpr (Cfg::HS) return (q >> 1) * 32 + 8 * g + 4 * (q & 1);
    else return q * 16 + 4 * g;
}

struct BlockGeo {
    int64_t t0;  // first token
    int Tv;      // valid tokens
};

__device__ __forceinline__ BlockGeo block_geo(const ScanParams &p, int blk) {
    BlockGeo g;
    g.t0 = (int64_t)blk * p.TB;
    const int64_t rem = p.T - g.t0;
    g.Tv = (int)(rem < (int64_t)p.TB ? rem : (int64_t)p.TB);
    return g;
}

// LDS carve-up
template <class Cfg, bool OUT>
struct Smem {
    unsigned char *bt, *ct, *gl, *wb, *xt, *ht, *ys, *phi, *raw;
    float *csr, *cs, *scale, *gam, *w, *ecs, *u, *isr, *tmp, *pend, *hmax, *aff;
    double *base;
    __device__ __forceinline__ explicit Smem(unsigned char *s) {
        unsigned char *q = s;
        if (OUT) {
            bt = q; q += Cfg::L_BT;
            ct = q; q += Cfg::L_CT;
            gl = q; q += Cfg::L_GL;
        } else {
            bt = ct = gl = nullptr;
        }
        wb = q; q += Cfg::L_WB;
        xt = q; q += Cfg::L_XT;
        if (OUT) { ht = q; q += Cfg::L_HT; ys = q; q += Cfg::L_Y; } else { ht = nullptr; ys = nullptr; }
        phi = q; q += Cfg::L_PHI;
        raw = nullptr;
        if (!OUT && Cfg::MV) { raw = q; q += Cfg::L_RAW; }
        float *f = (float *)q;
        csr = f;  // 16-byte aligned: (cos, sin) of pairs 2k, 2k + 1 are one f32x4
        cs = csr + Cfg::NP; scale = cs + Cfg::ROWS; gam = scale + Cfg::ROWS; w = gam + Cfg::ROWS;
        ecs = w + Cfg::ROWS; u = ecs + Cfg::ROWS; isr = u + Cfg::ROWS;
        tmp = isr + 2 * Cfg::ROWS;
        pend = tmp + 264; hmax = pend + Cfg::NP / 2;
        base = (double *)(q + Cfg::L_SC0);
        aff = (float *)(q + Cfg::L_SC);
    }
};

// eta_{-1} = dt_0 (1 - lambda_0) of the call's first token of batch b after the optional input
// activations: the weight of the carried previous B~ x^T in the first state.
__device__ __forceinline__ float eta_first(const ScanParams &p, int64_t b, int h) {
    float dt = p.dt[b * p.T * p.rsdt + h], lam = p.lam[b * p.T * p.rslam + h];
    if (p.flags & kFlagDtSoftplus) dt = softplus_f(dt + (p.dtbias ? p.dtbias[h] : 0.f));
    if (p.flags & kFlagLamSigmoid) lam = sigmoid_f(lam);
    return dt * (1.f - lam);
}
// Carried angle of pair i at the call's start (0 without a state or for a pair that does not rotate).
__device__ __forceinline__ double init_angle(const ScanParams &p, int64_t bh, int i) {
    return (p.ang0 && i < p.nr) ? (double)p.ang0[bh * p.nr + i] : 0.0;
}

// Per-workgroup constants: the sequence's base pointers and token strides.
struct WgCtx {
    int64_t b, bh;
    int h, cg, seg, p0, Pw, blk0, blk1;
    int R;      // rank (compile-time 1 on the SISO path)
    float invR; // 1 / R, to turn rows into tokens without an integer divide
    int Rx, Rz, Ry;             // ranks of x, z, y in memory: 1 when rank-free (MIMO projections)
    const void *xb, *Bb, *Cb;  // x, B, C at (b, token 0, h) (x offset by the column group)
    const float *thb, *dtb, *lamb, *ab;  // theta, dt, lambda, per-token A at (b, token 0, h)
    const void *zb;            // z at (b, token 0, h), offset by the column group
    void *yb;
    // row strides (elements between tokens) of x, B, C, theta, dt, lambda, A, z, y
    int sx, sb, sc, sth, sdt, slam, sa, sz, sy;
    float invN, eps;
    bool bcnorm, affine;
    bool rowscale;  // fp16 B~ / C~ rows get a power-of-two scale each (no norm, or gains / biases)
};

__device__ __forceinline__ int tok_of(int row, const WgCtx &c) {
    return (int)(((float)row + 0.5f) * c.invR);
}

// Issue the global loads of one block (nothing is converted so the loads stay in flight).
// PART selects what: kLoadXs = x, dt, lambda (and the per-token A), consumed by the staging of
// scalars and X^T; kLoadBc = B, C and theta, consumed by the prologue.  The rank-1 path issues
// the two parts at different points (each as soon as its registers are free); the other
// paths load everything with kLoadXs.
constexpr int kLoadXs = 1, kLoadBc = 2, kLoadAll = 3;
template <class Io, int PART = kLoadAll, class Cfg, bool WANT_C>
__device__ __forceinline__ void load_block(RawBlock<Cfg, WANT_C> &rb, const ScanParams &p, const WgCtx &c,
                                           const BlockGeo &g) {
    using ET = typename Io::T;
    const int tid = ltid(), lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, gq = lane >> 4;
    const int64_t T = p.T, H = p.H;
    const int N = p.N, P = p.P, N2 = p.N / 2;
    const int row = row_tile() * 16 + l16;
    const int64_t b = c.b;
    const int h = c.h;
    if constexpr (Cfg::VEC) {
        // SISO, N and P multiples of 8: row == token, 8 consecutive n per (lane, k step).
        // Uniform 64-bit block bases plus 32-bit per-lane byte offsets.
        const bool rv = row < g.Tv;
        if constexpr ((PART & kLoadBc) != 0) {
        // (B and C share their row stride on the 16-byte paths)
        const char *bbase = (const char *)c.Bb + (int64_t)g.t0 * c.sb * (int64_t)sizeof(ET);
        const char *cbase = (const char *)c.Cb + (int64_t)g.t0 * c.sb * (int64_t)sizeof(ET);
        const char *tbase = (const char *)c.thb + (int64_t)g.t0 * c.sth * 4;
        const uint32_t boff = (uint32_t)row * (uint32_t)(c.sb * sizeof(ET)) + (uint32_t)(8 * gq * sizeof(ET));
        const uint32_t toff = (uint32_t)row * (uint32_t)(c.sth * 4);
#pragma unroll
        for (int kk = 0; kk < Cfg::KS; ++kk) {
            const bool ok = rv && kk * 32 + 8 * gq < N;
#pragma unroll
            for (int q = 0; q < Cfg::BWV / 4; ++q) {
                u32x4_t vb = {0u, 0u, 0u, 0u}, vc = {0u, 0u, 0u, 0u};
                const uint32_t o = boff + (uint32_t)((kk * 32 + q * Cfg::XW) * sizeof(ET));
                if (ok) {
                    vb = *(const u32x4_t *)(bbase + o);
                    if constexpr (WANT_C) vc = *(const u32x4_t *)(cbase + o);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    rb.b[kk][q * 4 + k] = vb[k];
                    if constexpr (WANT_C) rb.c[kk][q * 4 + k] = vc[k];
                }
            }
            // angles of this lane's pairs: kk*16 + 4g + 0..3 (all four rotate or none: nr % 4 == 0)
            f32x4_t tv = {0.f, 0.f, 0.f, 0.f};
            const int po = pair_off<Cfg>(kk, gq);
            if (ok && po < p.nr) tv = *(const f32x4_t *)(tbase + toff + (uint32_t)(po * 4));
#pragma unroll
            for (int k = 0; k < 4; ++k) rb.th[kk * 4 + k] = tv[k];
        }
        }
        if constexpr ((PART & kLoadXs) != 0) {
        const char *xbase = (const char *)c.xb + (int64_t)g.t0 * c.sx * (int64_t)sizeof(ET);
#pragma unroll
        for (int m = 0; m < Cfg::XN / 4; ++m) {
            const int e = tid + 256 * m;
            const int xr = e / (Cfg::PP / Cfg::XW), pc = (e % (Cfg::PP / Cfg::XW)) * Cfg::XW;
            u32x4_t v = {0u, 0u, 0u, 0u};
            const uint32_t o = (uint32_t)xr * (uint32_t)(c.sx * sizeof(ET)) + (uint32_t)(pc * sizeof(ET));
            if (xr < g.Tv && pc < c.Pw) v = *(const u32x4_t *)(xbase + o);
#pragma unroll
            for (int k = 0; k < 4; ++k) rb.x[m * 4 + k] = v[k];
        }
        }
    } else if constexpr ((PART & kLoadXs) == 0) {
        // other paths: everything is loaded with the first part
    } else if constexpr (Cfg::MV) {
        // rank R in {2, 4, 8}: one token's B (C) is N*R contiguous values, n major, rank
        // minor; x is P*R.  16-byte vectors over every (token, vector) slot of the block;
        // slots past the block end or the padded n / p range load zeros.
        const int R = c.R;
        const int Tv = g.Tv;
        // x holds P values per token when rank-free (MIMO projection of x), P R otherwise
        const int Rx = Cfg::PJ ? c.Rx : R;
        const int vpt = (Cfg::NP * R) >> 3, xvpt = (Cfg::PP * Rx) >> 3;
        const float ivpt = 1.f / (float)vpt, ixvpt = 1.f / (float)xvpt;
        // (B and C share their row stride on the 16-byte paths)
        const char *bbase = (const char *)c.Bb + (int64_t)g.t0 * c.sb * (int64_t)sizeof(ET);
        const char *cbase = (const char *)c.Cb + (int64_t)g.t0 * c.sb * (int64_t)sizeof(ET);
#pragma unroll
        for (int m = 0; m < Cfg::NBV; ++m) {
            const int v = tid + 256 * m;
            const int tok = (int)(((float)v + 0.5f) * ivpt), o = v - tok * vpt;
            u32x4_t vb = {0u, 0u, 0u, 0u}, vc = {0u, 0u, 0u, 0u};
            if (tok < Tv && o * 8 < N * R) {
                const uint32_t off = (uint32_t)tok * (uint32_t)(c.sb * sizeof(ET)) + (uint32_t)(o * 16);
                vb = *(const u32x4_t *)(bbase + off);
                if constexpr (WANT_C) vc = *(const u32x4_t *)(cbase + off);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                rb.b[m][k] = vb[k];
                if constexpr (WANT_C) rb.c[m][k] = vc[k];
            }
        }
        const char *xbase = (const char *)c.xb + (int64_t)g.t0 * c.sx * (int64_t)sizeof(ET);
#pragma unroll
        for (int m = 0; m < Cfg::NXV; ++m) {
            const int v = tid + 256 * m;
            const int tok = (int)(((float)v + 0.5f) * ixvpt), o = v - tok * xvpt;
            u32x4_t vx = {0u, 0u, 0u, 0u};
            if (tok < Tv && o * 8 < c.Pw * Rx)
                vx = *(const u32x4_t *)(xbase + (uint32_t)tok * (uint32_t)(c.sx * sizeof(ET)) + (uint32_t)(o * 16));
#pragma unroll
            for (int k = 0; k < 4; ++k) rb.x[m * 4 + k] = vx[k];
        }
#pragma unroll
        for (int m = 0; m < Cfg::TN; ++m) {
            const int e = tid + 256 * m;
            const int tr = e / (Cfg::NP / 2), pc = e - tr * (Cfg::NP / 2);
            rb.th[m] = (tr < Tv && pc < p.nr) ? c.thb[(int64_t)(g.t0 + tr) * c.sth + pc] : 0.f;
        }
    } else {
        // general layout (rank R, any even N, any P): element loads
        const int R = c.R;
        const int tok = tok_of(row, c), r = row - tok * R;
        const bool rv = tok < g.Tv;
        const ET *bp = (const ET *)c.Bb + (int64_t)(g.t0 + tok) * c.sb + r;
        const ET *cp = (const ET *)c.Cb + (int64_t)(g.t0 + tok) * c.sc + r;
#pragma unroll
        for (int kk = 0; kk < Cfg::KS; ++kk) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int n = kk * 32 + 8 * gq + j;
                const bool ok = rv && n < N;
                rb.b[kk][j] = __float_as_uint(ok ? Io::ld(bp + (int64_t)n * R) : 0.f);
                if constexpr (WANT_C) rb.c[kk][j] = __float_as_uint(ok ? Io::ld(cp + (int64_t)n * R) : 0.f);
            }
        }
#pragma unroll
        for (int m = 0; m < Cfg::XN; ++m) {
            const int e = tid + 256 * m;
            const int xrow = e / Cfg::PP, pc = e - xrow * Cfg::PP;
            const int xt = tok_of(xrow, c), xrk = xrow - xt * R;
            float v = 0.f;
            if (xt < g.Tv && pc < c.Pw) {
                if (Cfg::PJ && p.mx)  // rank-free x expanded by the learned vector of rank xrk
                    v = Io::ld((const ET *)c.xb + (int64_t)(g.t0 + xt) * c.sx + pc) *
                        p.mx[((int64_t)h * R + xrk) * P + c.p0 + pc];
                else
                    v = Io::ld((const ET *)c.xb + (int64_t)(g.t0 + xt) * c.sx + (int64_t)pc * R + xrk);
            }
            rb.x[m] = __float_as_uint(v);
        }
#pragma unroll
        for (int m = 0; m < Cfg::TN; ++m) {
            const int e = tid + 256 * m;
            const int tr = e / (Cfg::NP / 2), pc = e - tr * (Cfg::NP / 2);
            rb.th[m] = (tr < g.Tv && pc < p.nr) ? c.thb[(int64_t)(g.t0 + tr) * c.sth + pc] : 0.f;
        }
    }
    if ((PART & kLoadXs) != 0 && wave == 0) {
        rb.dt = rb.lam = rb.dtn = rb.lamn = rb.av = 0.f;
        const float *db = c.dtb + (int64_t)g.t0 * c.sdt, *lb = c.lamb + (int64_t)g.t0 * c.slam;
        const uint32_t od = (uint32_t)lane * (uint32_t)c.sdt, ol = (uint32_t)lane * (uint32_t)c.slam;
        if (lane < g.Tv) {
            rb.dt = db[od];
            rb.lam = lb[ol];
            if (p.flags & kFlagAPerToken) rb.av = c.ab[(int64_t)(g.t0 + lane) * c.sa];
            if (g.t0 + lane + 1 < T) {
                rb.dtn = db[od + c.sdt];
                rb.lamn = lb[ol + c.slam];
            }
        }
    }
    (void)b;
    (void)h;
    (void)H;
    (void)P;
}

// Issue the loads of one block's gate input z (laid out like x and y).
template <class Io, class Cfg>
__device__ __forceinline__ void load_z(RawZ<Cfg> &rz, const ScanParams &p, const WgCtx &c, const BlockGeo &g) {
    using ET = typename Io::T;
    const int tid = ltid();
    const int R = c.R;
    // z at (b, token t0, h), offset by the column group like x
    const ET *zb = (const ET *)c.zb + (int64_t)g.t0 * c.sz;
    if constexpr (Cfg::VEC) {
#pragma unroll
        for (int m = 0; m < Cfg::XN / 4; ++m) {
            const int e = tid + 256 * m;
            const int zr = e / (Cfg::PP / Cfg::XW), pc = (e % (Cfg::PP / Cfg::XW)) * Cfg::XW;
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (zr < g.Tv && pc < c.Pw) v = *(const u32x4_t *)(zb + (int64_t)zr * c.sz + pc);
#pragma unroll
            for (int k = 0; k < 4; ++k) rz.w[m * 4 + k] = v[k];
        }
    } else if constexpr (Cfg::MV) {
        const int xvpt = (Cfg::PP * R) >> 3;
        const float ixvpt = 1.f / (float)xvpt;
#pragma unroll
        for (int m = 0; m < Cfg::NXV; ++m) {
            const int v = tid + 256 * m;
            const int tok = (int)(((float)v + 0.5f) * ixvpt), o = v - tok * xvpt;
            u32x4_t vz = {0u, 0u, 0u, 0u};
            if (tok < g.Tv && o * 8 < c.Pw * R) vz = *(const u32x4_t *)(zb + (int64_t)tok * c.sz + o * 8);
#pragma unroll
            for (int k = 0; k < 4; ++k) rz.w[m * 4 + k] = vz[k];
        }
    } else {
#pragma unroll
        for (int m = 0; m < Cfg::XN; ++m) {
            const int e = tid + 256 * m;
            const int zrow = e / Cfg::PP, pc = e - zrow * Cfg::PP;
            const int zt = tok_of(zrow, c), zrk = zrow - zt * R;
            float v = 0.f;
            if (zt < g.Tv && pc < c.Pw) v = Io::ld(zb + (int64_t)zt * c.sz + (int64_t)pc * R + zrk);
            rz.w[m] = __float_as_uint(v);
        }
    }
}

// Write the prefetched z into the y staging area at the positions the block's y values
// take (read back by the epilogue after two barriers; the area is free after the top one).
template <class Cfg, class Sm>
__device__ __forceinline__ void stage_z(const RawZ<Cfg> &rz, const Sm &sm, const WgCtx &c) {
    using ET = typename Cfg::ET;
    const int tid = ltid();
    ET *ys = (ET *)sm.ys;
    if constexpr (Cfg::VEC) {
#pragma unroll
        for (int m = 0; m < Cfg::XN / 4; ++m) {
            const int e = tid + 256 * m;
            const int zr = e / (Cfg::PP / Cfg::XW), pc = (e % (Cfg::PP / Cfg::XW)) * Cfg::XW;
            *(u32x4_t *)(ys + ys_off<Cfg>(zr, pc)) = u32x4_t{rz.w[m * 4], rz.w[m * 4 + 1], rz.w[m * 4 + 2], rz.w[m * 4 + 3]};
        }
    } else if constexpr (Cfg::MV) {
        const int R = c.R;
        const int xvpt = (Cfg::PP * R) >> 3;
        const float ixvpt = 1.f / (float)xvpt;
#pragma unroll
        for (int m = 0; m < Cfg::NXV; ++m) {
            const int v = tid + 256 * m;
            const int tok = (int)(((float)v + 0.5f) * ixvpt), o = v - tok * xvpt;
            if (tok * R >= Cfg::ROWS) continue;
            *(u32x4_t *)(ys + tok * Cfg::PP * R + o * 8) = u32x4_t{rz.w[m * 4], rz.w[m * 4 + 1], rz.w[m * 4 + 2], rz.w[m * 4 + 3]};
        }
    } else {
#pragma unroll
        for (int m = 0; m < Cfg::XN; ++m) {
            const int e = tid + 256 * m;
            const int zrow = e / Cfg::PP, pc = e - zrow * Cfg::PP;
            if constexpr (Cfg::BF) ys[ys_off<Cfg>(zrow, pc)] = (uint16_t)f2bf(__uint_as_float(rz.w[m]));
            else ys[ys_off<Cfg>(zrow, pc)] = __uint_as_float(rz.w[m]);
        }
    }
}

// decode the 8 B or C values of one k step
template <class Cfg, int BW>
__device__ __forceinline__ void raw8(const uint32_t (&w)[BW], float (&v)[8]) {
    if constexpr (Cfg::PACKED) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(w[k]);
    }
}

// two bf16 halves (half h of a and of b) -> one word, a's in the low half
__device__ __forceinline__ uint32_t pick_halves(uint32_t a, uint32_t b, int h) {
    return h ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

// Interleaved-rank path: regroup a block's raw B (and C) vectors per rank into
// [row][n] bf16 planes (pitch OPP), row = token * R + rank.  Every slot of the
// block is written (zeros past the block end and in the padded n range).
template <class Cfg, bool WANT_C>
__device__ __forceinline__ void stage_raw_bc(const RawBlock<Cfg, WANT_C> &rb, uint16_t *pb, uint16_t *pcp,
                                             const WgCtx &c) {
    const int tid = ltid();
    const int R = c.R;
    const int vpt = (Cfg::NP * R) >> 3;
    const float ivpt = 1.f / (float)vpt;
#pragma unroll
    for (int m = 0; m < Cfg::NBV; ++m) {
        const int v = tid + 256 * m;
        const int tok = (int)(((float)v + 0.5f) * ivpt), o = v - tok * vpt;
        if (tok * R >= Cfg::ROWS) continue;
        const int n0 = (o * 8) / R, row0 = tok * R;
        if (R == 2) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int off = (row0 + r) * Cfg::OPP + n0;
                *(u32x2_t *)(pb + off) = u32x2_t{pick_halves(rb.b[m][0], rb.b[m][1], r), pick_halves(rb.b[m][2], rb.b[m][3], r)};
                if constexpr (WANT_C)
                    *(u32x2_t *)(pcp + off) = u32x2_t{pick_halves(rb.c[m][0], rb.c[m][1], r), pick_halves(rb.c[m][2], rb.c[m][3], r)};
            }
        } else if (R == 4) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int off = (row0 + r) * Cfg::OPP + n0;
                *(uint32_t *)(pb + off) = pick_halves(rb.b[m][r >> 1], rb.b[m][(r >> 1) + 2], r & 1);
                if constexpr (WANT_C) *(uint32_t *)(pcp + off) = pick_halves(rb.c[m][r >> 1], rb.c[m][(r >> 1) + 2], r & 1);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int off = (row0 + r) * Cfg::OPP + n0;
                pb[off] = (uint16_t)((r & 1) ? (rb.b[m][r >> 1] >> 16) : (rb.b[m][r >> 1] & 0xffffu));
                if constexpr (WANT_C) pcp[off] = (uint16_t)((r & 1) ? (rb.c[m][r >> 1] >> 16) : (rb.c[m][r >> 1] & 0xffffu));
            }
        }
    }
}

// Stage 1 of a block: per-token scalars, angle partial sums and X^T into LDS.
// SISO: the angle running sum inside each wave's 16 rows is taken in
// registers (returned in `phi`); the 16-row totals go to LDS.  Ends with a barrier.
template <class Io, class Cfg, bool WANT_C, class Sm>
__device__ __forceinline__ void stage_scalars_x(RawBlock<Cfg, WANT_C> &rb, const Sm &sm, const ScanParams &p,
                                                const WgCtx &c, const BlockGeo &g) {
    const int tid = ltid(), lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15;
    if (wave == 0) {
        // the workgroup's other waves wait at the barrier below for this chain: it takes issue
        // priority over the co-resident workgroup's waves until its results are written
        __builtin_amdgcn_s_setprio(2);
        // log alpha, gamma, eta (next token's dt (1 - lambda); 0 after the last token), scale;
        // dt and lambda through the optional input activations, tokens past the end stay 0
        float dt = rb.dt, lam = rb.lam, dtn = rb.dtn, lamn = rb.lamn;
        if (p.flags & (kFlagDtSoftplus | kFlagLamSigmoid)) {
            const bool cur = lane < g.Tv, nxt = cur && g.t0 + lane + 1 < p.T;
            if (p.flags & kFlagDtSoftplus) {
                const float bias = p.dtbias ? p.dtbias[c.h] : 0.f;
                dt = cur ? softplus_f(dt + bias) : 0.f;
                dtn = nxt ? softplus_f(dtn + bias) : 0.f;
            }
            if (p.flags & kFlagLamSigmoid) {
                lam = cur ? sigmoid_f(lam) : 0.f;
                lamn = nxt ? sigmoid_f(lamn) : 0.f;
            }
        }
        const float la = dt * ((p.flags & kFlagAPerToken) ? rb.av : p.A[c.h]);
        const float ga = lam * dt;
        const float sc = ga + dtn * (1.f - lamn);
        const float cs = wave_incl_scan(la);
        const float cs_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
        sm.cs[lane] = cs;
        sm.scale[lane] = sc;
        sm.gam[lane] = ga;
        sm.ecs[lane] = __expf(cs);
        sm.w[lane] = __expf(cs_end - cs) * sc;
        if constexpr (Cfg::VEC) {
            // factored decay of the strictly causal tiles (s in an earlier 16-row tile than t):
            // exp(cs_t - cs_s) scale_s = exp(cs_t - cs_ref) * u_s, u_s = exp(cs_ref - cs_s) scale_s,
            // cs_ref the running sum at the last row of s's tile (both factors <= 1: cs falls)
            const float cref = __shfl(cs, lane | 15, 64);
            sm.u[lane] = __expf(cref - cs) * sc;
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (Cfg::VEC) {
        float *tt = (float *)sm.phi;  // [4 tiles][NP/2]
#pragma unroll
        for (int k = 0; k < Cfg::TN; ++k) rb.th[k] = row_incl_scan(rb.th[k]);
        if (l16 == 15) {
            const int gq = lane >> 4;
#pragma unroll
            for (int kk = 0; kk < Cfg::KS; ++kk)
                *(f32x4_t *)(tt + row_tile() * (Cfg::NP / 2) + pair_off<Cfg>(kk, gq)) =
                    f32x4_t{rb.th[kk * 4], rb.th[kk * 4 + 1], rb.th[kk * 4 + 2], rb.th[kk * 4 + 3]};
        }
    } else {
#pragma unroll
        for (int m = 0; m < Cfg::TN; ++m) {
            const int e = tid + 256 * m;
            const int tr = e / (Cfg::NP / 2), pc = e - tr * (Cfg::NP / 2);
            if (tr < Cfg::TOKS) ((float *)sm.phi)[tr * Cfg::PHP + pc] = rb.th[m];
        }
    }
    // x -> X^T [p][row]
    if constexpr (Cfg::MV) {
        const int R = c.R;
        uint16_t *xt = (uint16_t *)sm.xt;
        if (Cfg::PJ && p.mx) {
            // rank-free x: one vector holds 8 columns of a token; rank r of column q takes
            // x[q] mimo_x[h, r, q], rounded once to bf16, in the R consecutive rows of the token
            const int xvpt = Cfg::PP >> 3;
            const float ixvpt = 1.f / (float)xvpt;
            const float *mxh = p.mx + (int64_t)c.h * R * p.P + c.p0;
#pragma unroll
            for (int m = 0; m < Cfg::NXV; ++m) {
                const int v = tid + 256 * m;
                const int tok = (int)(((float)v + 0.5f) * ixvpt), o = v - tok * xvpt;
                if (tok * R >= Cfg::ROWS) continue;
                const int q0 = o * 8;
                const bool live = q0 < c.Pw;  // columns past the group width hold zeros
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t w = rb.x[m * 4 + (i >> 1)];
                    const float xv = __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
                    uint16_t *dst = xt + xt_off<Cfg>(q0 + i, tok * R);
                    for (int r = 0; r < R; ++r)
                        dst[r] = (uint16_t)f2bf(live ? xv * mxh[(int64_t)r * p.P + q0 + i] : 0.f);
                }
            }
        } else {
        // one vector holds 8 / R columns x R ranks: R consecutive rows of each column
        const int xvpt = (Cfg::PP * R) >> 3;
        const float ixvpt = 1.f / (float)xvpt;
#pragma unroll
        for (int m = 0; m < Cfg::NXV; ++m) {
            const int v = tid + 256 * m;
            const int tok = (int)(((float)v + 0.5f) * ixvpt), o = v - tok * xvpt;
            if (tok * R >= Cfg::ROWS) continue;
            const int p0 = (o * 8) / R, row0 = tok * R;
            if (R == 2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) *(uint32_t *)(xt + xt_off<Cfg>(p0 + i, row0)) = rb.x[m * 4 + i];
            } else if (R == 4) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    *(u32x2_t *)(xt + xt_off<Cfg>(p0 + i, row0)) = u32x2_t{rb.x[m * 4 + 2 * i], rb.x[m * 4 + 2 * i + 1]};
            } else {
                *(u32x4_t *)(xt + xt_off<Cfg>(p0, row0)) = u32x4_t{rb.x[m * 4], rb.x[m * 4 + 1], rb.x[m * 4 + 2], rb.x[m * 4 + 3]};
            }
        }
        }
    } else if constexpr (Cfg::VEC) {
#pragma unroll
        for (int m = 0; m < Cfg::XN / 4; ++m) {
            const int e = tid + 256 * m;
            const int xr = e / (Cfg::PP / Cfg::XW), pc = (e % (Cfg::PP / Cfg::XW)) * Cfg::XW;
            // the XW columns pc .. pc + XW - 1 (pc a multiple of XW <= 8) share their swizzle:
            // one base address, constant offsets
            if constexpr (Cfg::BF) {
                uint16_t *xt = (uint16_t *)sm.xt + xt_off<Cfg>(pc, xr);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    xt[(2 * k) * Cfg::RPP] = (uint16_t)(rb.x[m * 4 + k] & 0xffffu);
                    xt[(2 * k + 1) * Cfg::RPP] = (uint16_t)(rb.x[m * 4 + k] >> 16);
                }
            } else {
                float *xt = (float *)sm.xt + xt_off<Cfg>(pc, xr);
#pragma unroll
                for (int k = 0; k < 4; ++k) xt[k * Cfg::RPP] = __uint_as_float(rb.x[m * 4 + k]);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < Cfg::XN; ++m) {
            const int e = tid + 256 * m;
            const int xrow = e / Cfg::PP, pc = e - xrow * Cfg::PP;
            const float v = __uint_as_float(rb.x[m]);
            if constexpr (Cfg::BF) ((uint16_t *)sm.xt)[xt_off<Cfg>(pc, xrow)] = (uint16_t)f2bf(v);
            else ((float *)sm.xt)[xt_off<Cfg>(pc, xrow)] = v;
        }
    }
    lds_barrier();
}

// Stage 2 (general path only): running angle over the table (segmented scan per pair).  Ends with a barrier.
template <class Cfg, class Sm>
__device__ __forceinline__ void stage_angles_table(const Sm &sm, const ScanParams &p, const BlockGeo &g) {
    const int tid = ltid();
    const int N2 = p.N / 2;
    const int Tv = g.Tv;
    float *phi = (float *)sm.phi;
    int nseg = 256 / N2;
    if (nseg > Tv) nseg = Tv;
    if (nseg < 1) nseg = 1;
    const int seglen = (Tv + nseg - 1) / nseg;
    const int i = tid % N2, sg = tid / N2;
    if (sg < nseg) {
        const int ta = sg * seglen, tb = min(Tv, ta + seglen);
        float acc = 0.f;
        for (int t = ta; t < tb; ++t) {
            acc += phi[t * Cfg::PHP + i];
            phi[t * Cfg::PHP + i] = acc;
        }
        sm.tmp[sg * N2 + i] = acc;
    }
    lds_barrier();
    if (sg < nseg && sg > 0) {
        float off = 0.f;
        for (int k = 0; k < sg; ++k) off += sm.tmp[k * N2 + i];
        const int ta = sg * seglen, tb = min(Tv, ta + seglen);
        for (int t = ta; t < tb; ++t) phi[t * Cfg::PHP + i] += off;
    }
    lds_barrier();
}

// Block angle totals per pair (and their cos/sin) for the carry.  Reads the
// angle data of stage 1/2; the results are consumed after a later barrier.
template <class Cfg, class Sm>
__device__ __forceinline__ void block_angle_totals(const Sm &sm, const ScanParams &p, const BlockGeo &g, int wave0 = 0) {
    const int tid = ltid() - 64 * wave0;  // pairs on the lanes of wave `wave0`
    const int N2 = p.N / 2;
    if (tid >= 0 && tid < N2) {
        float a;
        if constexpr (Cfg::VEC) {
            const float *tt = (const float *)sm.phi;
            a = tt[tid] + tt[Cfg::NP / 2 + tid] + tt[2 * (Cfg::NP / 2) + tid] + tt[3 * (Cfg::NP / 2) + tid];
        } else {
            a = ((const float *)sm.phi)[(g.Tv - 1) * Cfg::PHP + tid];
        }
        const f32x2_t sc_ = sincos_acc(a);
        sm.pend[tid] = a;
        *(f32x2_t *)(sm.csr + 2 * tid) = f32x2_t{sc_[1], sc_[0]};
    }
}

// (cos, sin) of the padded pairs N/2 .. NP/2 - 1: (1, 0), never rewritten (their state rows are 0)
template <class Cfg, class Sm>
__device__ __forceinline__ void init_pad_pairs(const Sm &sm, const ScanParams &p) {
    const int tid = ltid();
    if (tid >= p.N / 2 && tid < Cfg::NP / 2) *(f32x2_t *)(sm.csr + 2 * tid) = f32x2_t{1.f, 0.f};
}

// Stage 3: B~ (and C~) for the rows this lane owns: norm, gains and biases, rotation by the
// block-local angle.  Writes (w B~)^T [n][row] to LDS (bf16 hi/lo, or fp32) and, in output
// mode, B~ [row][n] (fp16 times the row scale, or fp32) and returns the C~ fragments (fp16
// times the row scale, or fp32); the inverse row scales go to sm.isr when c.rowscale.  With
// `final_row` (the call's last block, in the workgroup that writes the final state) the lanes
// of the last token's rows also write that token's B~, rotated into the global frame, to the
// final state's prev_B.
template <class Io, class Cfg, bool WANT_C, class Frag, class Sm>
__device__ __forceinline__ void stage_prologue(const RawBlock<Cfg, WANT_C> &rb, const Sm &sm, const ScanParams &p,
                                               const WgCtx &c, const BlockGeo &g, Frag (&ct)[Cfg::KS],
                                               bool final_row) {
    constexpr int KS = Cfg::KS;
    const int tid = ltid(), lane = tid & 63;
    const int l16 = lane & 15, gq = lane >> 4;
    const int N = p.N;
    const int R = Cfg::VEC ? 1 : c.R;
    const int row = row_tile() * 16 + l16;
    const int tok = Cfg::VEC ? row : tok_of(row, c);
    const int r = row - tok * R;
    const bool rv = tok < g.Tv;
    // raw B / C words of this lane's row: registers, or (interleaved ranks) the regrouped planes
    using RB = RawBlock<Cfg, WANT_C>;
    uint32_t bw[KS][RB::BW], cw[WANT_C ? KS : 1][RB::BW];
    if constexpr (Cfg::MV) {
        const uint16_t *pb = WANT_C ? (const uint16_t *)sm.bt : (const uint16_t *)sm.raw;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int off = row * Cfg::OPP + kk * 32 + 8 * gq;
            const u32x4_t v = *(const u32x4_t *)(pb + off);
#pragma unroll
            for (int k = 0; k < 4; ++k) bw[kk][k] = v[k];
            if constexpr (WANT_C) {
                const u32x4_t u = *(const u32x4_t *)((const uint16_t *)sm.bt + Cfg::BT_PLANE + off);
#pragma unroll
                for (int k = 0; k < 4; ++k) cw[kk][k] = u[k];
            }
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int k = 0; k < RB::BW; ++k) {
                bw[kk][k] = rb.b[kk][k];
                if constexpr (WANT_C) cw[kk][k] = rb.c[kk][k];
            }
    }
    float ssb = 0.f, ssc = 0.f;
    if constexpr (Cfg::PACKED) {
        // packed bf16 pairs: one dot2 per two squares
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                ssb = sumsq2_bf16(bw[kk][k], ssb);
                if constexpr (WANT_C) ssc = sumsq2_bf16(cw[kk][k], ssc);
            }
    } else {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float vb[8], vc[8];
            raw8<Cfg>(bw[kk], vb);
            if constexpr (WANT_C) raw8<Cfg>(cw[kk], vc);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                ssb = fmaf(vb[j], vb[j], ssb);
                if constexpr (WANT_C) ssc = fmaf(vc[j], vc[j], ssc);
            }
        }
    }
    ssb = rows_sum4(ssb);
    if constexpr (WANT_C) ssc = rows_sum4(ssc);
    // norm factors; rows past the block end are zero
    const float rsb = rv ? (c.bcnorm ? __builtin_amdgcn_rsqf(fmaf(ssb, c.invN, c.eps)) : 1.f) : 0.f;
    const float rsc = rv ? (c.bcnorm ? __builtin_amdgcn_rsqf(fmaf(ssc, c.invN, c.eps)) : 1.f) : 0.f;
    const float wt = sm.w[tok];  // zero past the block end
    // angle offsets of the earlier 16-row tiles (SISO path; the tile index is wave-uniform)
    f32x4_t phoff[KS];
    if constexpr (Cfg::VEC) {
        const float *tt = (const float *)sm.phi;
        const int rtile = row_tile();
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) phoff[kk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int w2 = 0; w2 < rtile; ++w2)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) phoff[kk] += *(const f32x4_t *)(tt + w2 * (Cfg::NP / 2) + pair_off<Cfg>(kk, gq));
    }
    // normalised values with gains and biases of one k step (8 components of the row)
    auto prep = [&](int kk, float (&vb)[8], float (&vc)[8]) {
        raw8<Cfg>(bw[kk], vb);
        if constexpr (WANT_C) raw8<Cfg>(cw[kk], vc);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            vb[j] *= rsb;
            if constexpr (WANT_C) vc[j] *= rsc;
        }
        if constexpr (Cfg::VEC) {
            if (c.affine && rv) {
                // gains (with the norm) and this head's biases, staged in LDS at kernel start
                const int n0 = kk * 32 + 8 * gq;
                const f32x4_t g0 = *(const f32x4_t *)(sm.aff + n0), g1 = *(const f32x4_t *)(sm.aff + n0 + 4);
                const f32x4_t b0 = *(const f32x4_t *)(sm.aff + 2 * Cfg::NP + n0);
                const f32x4_t b1 = *(const f32x4_t *)(sm.aff + 2 * Cfg::NP + n0 + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vb[j] = fmaf(vb[j], g0[j], b0[j]);
                    vb[j + 4] = fmaf(vb[j + 4], g1[j], b1[j]);
                }
                if constexpr (WANT_C) {
                    const f32x4_t h0 = *(const f32x4_t *)(sm.aff + Cfg::NP + n0), h1 = *(const f32x4_t *)(sm.aff + Cfg::NP + n0 + 4);
                    const f32x4_t d0 = *(const f32x4_t *)(sm.aff + 3 * Cfg::NP + n0);
                    const f32x4_t d1 = *(const f32x4_t *)(sm.aff + 3 * Cfg::NP + n0 + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        vc[j] = fmaf(vc[j], h0[j], d0[j]);
                        vc[j + 4] = fmaf(vc[j + 4], h1[j], d1[j]);
                    }
                }
            }
        } else if (c.affine && rv) {
            // gains (with the norm) and per-(head, rank) biases
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int n = kk * 32 + 8 * gq + j;
                if (n < N) {
                    if (c.bcnorm && p.bnw) vb[j] *= p.bnw[n];
                    if (p.bbias) vb[j] += p.bbias[((int64_t)c.h * R + r) * N + n];
                    if constexpr (WANT_C) {
                        if (c.bcnorm && p.cnw) vc[j] *= p.cnw[n];
                        if (p.cbias) vc[j] += p.cbias[((int64_t)c.h * R + r) * N + n];
                    }
                }
            }
        }
    };
    // fp16 row scales: a power of two that maps the row's largest |component| into [2^11, 2^12)
    // (a rotated component is at most sqrt(2) times that); 1 for normalised rows without gains
    // or biases, whose components are at most sqrt(N)
    float sgb = 1.f, sgc = 1.f;
    if constexpr (Cfg::F16 && WANT_C) {
        if (c.rowscale) {
            float mb = 0.f, mc = 0.f;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                float vb[8], vc[8];
                prep(kk, vb, vc);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    mb = fmaxf(mb, fabsf(vb[j]));
                    mc = fmaxf(mc, fabsf(vc[j]));
                }
            }
            mb = rows_max4(mb);
            mc = rows_max4(mc);
            float ib, ic;
            pow2_scale<12>(mb, sgb, ib);
            pow2_scale<12>(mc, sgc, ic);
            if (gq == 0) {
                sm.isr[row] = ib;
                sm.isr[Cfg::ROWS + row] = ic;
            }
        }
    }
    const bool last_tok = final_row && rv && tok == g.Tv - 1;
    // the rotated B~ (ob) and C~ (oc) components kk*32 + 8g .. + 7 of this row -> the B~, C~ and
    // (w B~)^T planes (and, off the column-owned path, the C~ fragment of step kk)
    auto write_planes = [&](int kk, const float (&ob)[8], const float (&oc)[8]) {
        // the 8 components n0 .. n0 + 7 share their swizzle in the (w B~)^T plane
        const int n0 = kk * 32 + 8 * gq;
        if constexpr (Cfg::BF) {
            uint32_t wh[4], wl[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) split2(ob[2 * k] * wt, ob[2 * k + 1] * wt, wh[k], wl[k]);
            if constexpr (WANT_C) {
                const int off = row * Cfg::OPP + n0;
                u32x4_t bw4, cw4;
                // (the N = 128 variants, at the whole register file, keep the one multiplying path:
                // the branch measured slower there)
                if (Cfg::NP > 64 || c.rowscale) {
                    bw4 = u32x4_t{pack_f16(ob[0] * sgb, ob[1] * sgb), pack_f16(ob[2] * sgb, ob[3] * sgb),
                                  pack_f16(ob[4] * sgb, ob[5] * sgb), pack_f16(ob[6] * sgb, ob[7] * sgb)};
                    cw4 = u32x4_t{pack_f16(oc[0] * sgc, oc[1] * sgc), pack_f16(oc[2] * sgc, oc[3] * sgc),
                                  pack_f16(oc[4] * sgc, oc[5] * sgc), pack_f16(oc[6] * sgc, oc[7] * sgc)};
                } else {
                    // unit row scales (normalised rows without gains or biases): no multiplies
                    bw4 = u32x4_t{pack_f16(ob[0], ob[1]), pack_f16(ob[2], ob[3]), pack_f16(ob[4], ob[5]), pack_f16(ob[6], ob[7])};
                    cw4 = u32x4_t{pack_f16(oc[0], oc[1]), pack_f16(oc[2], oc[3]), pack_f16(oc[4], oc[5]), pack_f16(oc[6], oc[7])};
                }
                *(u32x4_t *)((uint16_t *)sm.bt + off) = bw4;
                if constexpr (Cfg::COL) *(u32x4_t *)((uint16_t *)sm.ct + off) = cw4;  // read by every wave
                else ct[kk].v = cw4;
            }
            uint16_t *wb = (uint16_t *)sm.wb + tr_off<Cfg>(n0, row);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                wb[(2 * k) * Cfg::RPP] = (uint16_t)(wh[k] & 0xffffu);
                wb[(2 * k + 1) * Cfg::RPP] = (uint16_t)(wh[k] >> 16);
                wb[Cfg::WB_PLANE + (2 * k) * Cfg::RPP] = (uint16_t)(wl[k] & 0xffffu);
                wb[Cfg::WB_PLANE + (2 * k + 1) * Cfg::RPP] = (uint16_t)(wl[k] >> 16);
            }
        } else {
            if constexpr (WANT_C) {
                const int off = row * Cfg::OPP + n0;
                float *bt = (float *)sm.bt;
                *(f32x4_t *)(bt + off) = f32x4_t{ob[0], ob[1], ob[2], ob[3]};
                *(f32x4_t *)(bt + off + 4) = f32x4_t{ob[4], ob[5], ob[6], ob[7]};
#pragma unroll
                for (int j = 0; j < 8; ++j) ct[kk].v[j] = oc[j];
            }
            float *wb = (float *)sm.wb + tr_off<Cfg>(n0, row);
#pragma unroll
            for (int j = 0; j < 8; ++j) wb[j * Cfg::RPP] = ob[j] * wt;
        }
    };
    if constexpr (Cfg::HS) {
        // half-split pairing: component n = k2*32 + 8g + j (step k2 < KS/2) pairs with n + N/2
        // (step k2 + KS/2, same slot); pair n's angle is in angle group 2 k2 + j / 4
#pragma unroll
        for (int k2 = 0; k2 < KS / 2; ++k2) {
            float vb0[8], vc0[8], vb1[8], vc1[8];
            prep(k2, vb0, vc0);
            prep(k2 + KS / 2, vb1, vc1);
            float ob0[8], oc0[8], ob1[8], oc1[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int q = 2 * k2 + (j >> 2);
                float sn, cn;
                fast_sincos(rb.th[q * 4 + (j & 3)] + phoff[q][j & 3], sn, cn);
                const float u = vb0[j], v = vb1[j];
                ob0[j] = u * cn - v * sn;
                ob1[j] = u * sn + v * cn;
                if constexpr (WANT_C) {
                    const float uc = vc0[j], vcc = vc1[j];
                    oc0[j] = uc * cn - vcc * sn;
                    oc1[j] = uc * sn + vcc * cn;
                }
            }
            if (last_tok) {
                // the carried B~ of the call's last token, rotated into the global frame
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int n = k2 * 32 + 8 * gq + j;
                    float sn, cn;
                    fast_sincos((float)wrap_2pi(sm.base[n]), sn, cn);
                    const float u = ob0[j], v = ob1[j];
                    p.pB1[(c.bh * N + n) * R + r] = u * cn - v * sn;
                    p.pB1[(c.bh * N + n + N / 2) * R + r] = u * sn + v * cn;
                }
            }
            write_planes(k2, ob0, oc0);
            write_planes(k2 + KS / 2, ob1, oc1);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float vb[8], vc[8];
            prep(kk, vb, vc);
            float ob[8], oc[8];
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) {
                const int n = kk * 32 + 8 * gq + 2 * jp;
                float ang;
                if constexpr (Cfg::VEC) ang = rb.th[kk * 4 + jp] + phoff[kk][jp];
                else ang = (rv && n < N) ? ((const float *)sm.phi)[tok * Cfg::PHP + n / 2] : 0.f;
                float sn, cn;
                fast_sincos(ang, sn, cn);
                const float u = vb[2 * jp], v = vb[2 * jp + 1];
                ob[2 * jp] = u * cn - v * sn;
                ob[2 * jp + 1] = u * sn + v * cn;
                if constexpr (WANT_C) {
                    const float uc = vc[2 * jp], vcc = vc[2 * jp + 1];
                    oc[2 * jp] = uc * cn - vcc * sn;
                    oc[2 * jp + 1] = uc * sn + vcc * cn;
                }
            }
            if (last_tok) {
                // the carried B~ of the call's last token: from the block frame to the global frame
                // (the running angle at this block's start)
#pragma unroll
                for (int jp = 0; jp < 4; ++jp) {
                    const int n = kk * 32 + 8 * gq + 2 * jp;
                    if (n < N) {
                        float sn, cn;
                        fast_sincos((float)wrap_2pi(sm.base[n / 2]), sn, cn);
                        const float u = ob[2 * jp], v = ob[2 * jp + 1];
                        p.pB1[(c.bh * N + n) * R + r] = u * cn - v * sn;
                        p.pB1[(c.bh * N + n + 1) * R + r] = u * sn + v * cn;
                    }
                }
            }
            write_planes(kk, ob, oc);
        }
    }
    (void)tid;
}

// State tiles of this wave: tile e = wave + 4m -> (nt = e / PT, pt = e % PT);
// fragment slot i of lane l holds element (n = nt*16 + 4(l/16) + i, p = pt*16 + l%16).
template <class Cfg>
__device__ __forceinline__ bool state_tile(int m, int &nt, int &pt) {
    const int e = (ltid() >> 6) + 4 * m;
    nt = e / Cfg::PT;
    pt = e - nt * Cfg::PT;
    return e < Cfg::PT * Cfg::NT;
}

// acc += (w B~)^T X for this wave's state tiles
template <class Cfg, class Sm>
__device__ __forceinline__ void mfma_state(const Sm &sm, f32x4_t (&acc)[Cfg::TPW]) {
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int m = 0; m < Cfg::TPW; ++m) {
        int nt, pt;
        if (!state_tile<Cfg>(m, nt, pt)) continue;
#pragma unroll
        for (int kk = 0; kk < Cfg::ROWS / 32; ++kk) {
            const int wo = tr_off<Cfg>(nt * 16 + l16, kk * 32 + 8 * gq);
            const int xo = xt_off<Cfg>(pt * 16 + l16, kk * 32 + 8 * gq);
            if constexpr (Cfg::BF) {
                FragHL wf;
                wf.hi = *(const u32x4_t *)((const uint16_t *)sm.wb + wo);
                wf.lo = *(const u32x4_t *)((const uint16_t *)sm.wb + Cfg::WB_PLANE + wo);
                const u32x4_t xb = *(const u32x4_t *)((const uint16_t *)sm.xt + xo);
                acc[m] = mma(wf, xb, acc[m]);
            } else {
                FragF wf, xb;
                const float *wp = (const float *)sm.wb + wo, *xp = (const float *)sm.xt + xo;
                const f32x4_t w0 = *(const f32x4_t *)wp, w1 = *(const f32x4_t *)(wp + 4);
                const f32x4_t x0 = *(const f32x4_t *)xp, x1 = *(const f32x4_t *)(xp + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wf.v[j] = w0[j]; wf.v[j + 4] = w1[j];
                    xb.v[j] = x0[j]; xb.v[j + 4] = x1[j];
                }
                acc[m] = mma(wf, xb, acc[m]);
            }
        }
    }
}

// rotate the pairs (slot 0, 1) and (slot 2, 3) of a state fragment by -angle (cos c, sin s)
__device__ __forceinline__ void rot_neg(f32x4_t &v, float c0, float s0, float c1, float s1) {
    const float u0 = v[0], v0 = v[1], u1 = v[2], v1 = v[3];
    v[0] = u0 * c0 + v0 * s0;
    v[1] = -u0 * s0 + v0 * c0;
    v[2] = u1 * c1 + v1 * s1;
    v[3] = -u1 * s1 + v1 * c1;
}
// Half-split pairing: slot i of a (row n) pairs with slot i of b (row n + N/2); rotation by
// -angle_i with (cos, sin) of pairs n .. n+3 in (cs01, cs23) = (c0, s0, c1, s1), (c2, s2, c3, s3).
__device__ __forceinline__ void rot_neg_hs(f32x4_t &a, f32x4_t &b, const f32x4_t &cs01, const f32x4_t &cs23) {
    const float cc[4] = {cs01[0], cs01[2], cs23[0], cs23[2]}, ss[4] = {cs01[1], cs01[3], cs23[1], cs23[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float u = a[i], v = b[i];
        a[i] = u * cc[i] + v * ss[i];
        b[i] = -u * ss[i] + v * cc[i];
    }
}

// H <- Rot(-Phi) H for this wave's state fragments, with (cos, sin) of Phi per pair in sm.csr.
template <class Cfg, class Sm>
__device__ __forceinline__ void rot_state(const Sm &sm, f32x4_t (&hs)[Cfg::TPW]) {
    const int gq = (threadIdx.x & 63) >> 4;
    if constexpr (Cfg::HS) {
#pragma unroll
        for (int m = 0; m < Cfg::HSM; ++m) {
            int nt, pt;
            state_tile<Cfg>(m, nt, pt);
            const int n0 = nt * 16 + 4 * gq;  // pairs n0 .. n0 + 3 (rows n0 + i and n0 + i + N/2)
            const f32x4_t cs01 = *(const f32x4_t *)(sm.csr + 2 * n0), cs23 = *(const f32x4_t *)(sm.csr + 2 * n0 + 4);
            rot_neg_hs(hs[m], hs[m + Cfg::HSM], cs01, cs23);
        }
    } else {
#pragma unroll
        for (int m = 0; m < Cfg::TPW; ++m) {
            int nt, pt;
            if (!state_tile<Cfg>(m, nt, pt)) continue;
            const int pr = (nt * 16 + 4 * gq) >> 1;  // pairs pr, pr + 1 (pr even)
            const f32x4_t cs4 = *(const f32x4_t *)(sm.csr + 2 * pr);
            rot_neg(hs[m], cs4[0], cs4[1], cs4[2], cs4[3]);
        }
    }
}

// Carry update:  H <- Rot(-Phi) (decay H + S), with the matrix cores adding S
// into the decayed state in place.
template <class Cfg, class Sm>
__device__ __forceinline__ void carry_block(const Sm &sm, f32x4_t (&hs)[Cfg::TPW], float decay) {
#pragma unroll
    for (int m = 0; m < Cfg::TPW; ++m) hs[m] *= decay;
    mfma_state<Cfg>(sm, hs);
    rot_state<Cfg>(sm, hs);
}

// H fragments -> the H^T [p][n] plane in LDS, 4 consecutive n per lane: fp16 times a power of
// two that maps the block's largest |H| (the maxima the waves left in sm.hmax) into
// [2^13, 2^14), or fp32.  Returns the inverse of that scale (1 for fp32).
template <class Cfg, class Sm>
__device__ __forceinline__ float write_ht(const Sm &sm, const f32x4_t (&hs)[Cfg::TPW]) {
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, gq = lane >> 4;
    float sc = 1.f, inv = 1.f;
    if constexpr (Cfg::F16) {
        const f32x4_t m4 = *(const f32x4_t *)sm.hmax;
        pow2_scale<14>(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])), sc, inv);
    }
#pragma unroll
    for (int m = 0; m < Cfg::TPW; ++m) {
        int nt, pt;
        if (!state_tile<Cfg>(m, nt, pt)) continue;
        const int off = (pt * 16 + l16) * Cfg::OPP + nt * 16 + 4 * gq;
        if constexpr (Cfg::F16) {
            *(u32x2_t *)((uint16_t *)sm.ht + off) =
                u32x2_t{pack_f16(hs[m][0] * sc, hs[m][1] * sc), pack_f16(hs[m][2] * sc, hs[m][3] * sc)};
        } else {
            *(f32x4_t *)((float *)sm.ht + off) = hs[m];
        }
    }
    return inv;
}

// Largest |component| over the 64 lanes of a wave (values >= 0; every lane active): inclusive
// max inside rows of 16, then across rows as in wave_incl_scan; lane 63's value, broadcast.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// This wave's largest |H| -> sm.hmax[wave], read by every wave's next write_ht (fp16 path).
template <class Cfg, class Sm>
__device__ __forceinline__ void publish_hmax(const Sm &sm, const f32x4_t (&hs)[Cfg::TPW]) {
    if constexpr (Cfg::F16) {
        float m = 0.f;
#pragma unroll
        for (int k = 0; k < Cfg::TPW; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(hs[k][i]));
        m = wave_max_nonneg(m);
        if ((threadIdx.x & 63) == 0) sm.hmax[ltid() >> 6] = m;
    }
}

// workgroup -> (sequence, column group, segment); the segments of one
// (sequence, column group) share an XCD when the count allows it
__device__ __forceinline__ void wg_map(int64_t nbh, int ncg, int nsegk, int64_t &bh, int &cg, int &seg) {
    const int64_t bid = blockIdx.x;
    const int64_t nq = nbh * ncg;
    int64_t q;
    if ((nq & 7) == 0) {
        const int64_t xcd = bid & 7, k = bid >> 3;
        q = xcd + 8 * (k / nsegk);
        seg = (int)(k % nsegk);
    } else {
        q = bid / nsegk;
        seg = (int)(bid % nsegk);
    }
    bh = q / ncg;
    cg = (int)(q - bh * ncg);
}

template <class Cfg>
__device__ __forceinline__ WgCtx make_ctx(const ScanParams &p, int nsegk, int bpu) {
    WgCtx c;
    wg_map(p.B * p.H, p.ncg, nsegk, c.bh, c.cg, c.seg);
    c.b = c.bh / p.H;
    c.h = (int)(c.bh - c.b * p.H);
    c.p0 = c.cg * Cfg::PP;
    c.Pw = min(Cfg::PP, p.P - c.p0);
    c.blk0 = c.seg * bpu;
    c.blk1 = min(p.nblk, c.blk0 + bpu);
    c.R = Cfg::VEC ? 1 : p.R;
    c.invR = 1.f / (float)c.R;
    using ET = typename Cfg::ET;
    const int64_t row0 = c.b * p.T;  // row of (b, token 0)
    c.Rx = p.mx ? 1 : c.R;
    c.Rz = p.mz ? 1 : c.R;
    c.Ry = p.mo ? 1 : c.R;
    c.sx = (int)p.rsx;
    c.sb = (int)p.rsb;
    c.sc = (int)p.rsc;
    c.sth = (int)p.rsth;
    c.sdt = (int)p.rsdt;
    c.slam = (int)p.rslam;
    c.sa = (int)p.rsa;
    c.sz = (int)p.rsz;
    c.sy = (int)p.rsy;
    c.xb = (const ET *)p.x + row0 * p.rsx + ((int64_t)c.h * p.P + c.p0) * c.Rx;
    c.Bb = (const ET *)p.Bm + row0 * p.rsb + (int64_t)c.h * p.N * c.R;
    c.Cb = (const ET *)p.Cm + row0 * p.rsc + (int64_t)c.h * p.N * c.R;
    c.thb = p.theta + row0 * p.rsth + (int64_t)c.h * p.nr;
    c.dtb = p.dt + row0 * p.rsdt + c.h;
    c.lamb = p.lam + row0 * p.rslam + c.h;
    c.ab = p.A + row0 * p.rsa + c.h;
    c.zb = (const ET *)p.z + row0 * p.rsz + ((int64_t)c.h * p.P + c.p0) * c.Rz;
    c.yb = (ET *)p.y + row0 * p.rsy + ((int64_t)c.h * p.P + c.p0) * c.Ry;
    c.invN = 1.f / (float)p.N;
    c.eps = p.eps;
    c.bcnorm = (p.flags & kFlagNorm) != 0;
    c.affine = (c.bcnorm && (p.bnw || p.cnw)) || p.bbias || p.cbias;
    // normalised rows without gains or biases have |components| <= sqrt(N) <= 11.4: fp16 as is
    c.rowscale = Cfg::F16 && !(c.bcnorm && !c.affine);
    M3_DCHECK(p, c.b < p.B && c.h < p.H && c.cg < p.ncg && c.seg < nsegk && c.blk0 < c.blk1 &&
                     c.blk1 <= p.nblk && c.Pw >= 1 && c.p0 + c.Pw <= p.P);
    return c;
}

// Rank-1 path: gains and this head's biases into LDS ([4][NP]; 1 and 0 when absent
// or past N).  Read after the next barrier.
template <class Cfg, class Sm>
__device__ __forceinline__ void stage_affine(const Sm &sm, const ScanParams &p, const WgCtx &c) {
    if constexpr (Cfg::VEC) {
        const int tid = ltid();
        if (tid < Cfg::NP) {
            const int n = tid;
            const bool in = n < p.N;
            const bool g = c.bcnorm;  // gains apply only together with the norm
            sm.aff[n] = (in && g && p.bnw) ? p.bnw[n] : 1.f;
            sm.aff[Cfg::NP + n] = (in && g && p.cnw) ? p.cnw[n] : 1.f;
            sm.aff[2 * Cfg::NP + n] = (in && p.bbias) ? p.bbias[(int64_t)c.h * p.N + n] : 0.f;
            sm.aff[3 * Cfg::NP + n] = (in && p.cbias) ? p.cbias[(int64_t)c.h * p.N + n] : 0.f;
        }
    }
}

// ============================================================ state kernel
template <class Io, int NP, int PP, int MODE, bool PJ, bool HS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 4))) void seg_state_kernel(ScanParams p) {
    using Cfg = SegCfg<Io, NP, PP, MODE, true, PJ, HS>;
    constexpr bool VEC = Cfg::VEC;
    using Frag = typename std::conditional<Cfg::BF, FragH, FragF>::type;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const Smem<Cfg, false> sm(smem);
    const WgCtx c = make_ctx<Cfg>(p, p.nsub, p.sbps);  // c.seg: the state sub-segment
    const int tid = ltid(), lane = tid & 63;
    const int N2 = p.N / 2;

    f32x4_t sagg[Cfg::TPW];
#pragma unroll
    for (int m = 0; m < Cfg::TPW; ++m) sagg[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (tid < N2) sm.base[tid] = 0.0;
    init_pad_pairs<Cfg>(sm, p);
    float lsum = 0.f;
    Frag ct_unused[Cfg::KS];

    stage_affine<Cfg>(sm, p, c);
    RawBlock<Cfg, false> rb;
    BlockGeo g = block_geo(p, c.blk0);
    load_block<Io>(rb, p, c, g);
    if constexpr (Cfg::MV) stage_raw_bc<Cfg>(rb, (uint16_t *)sm.raw, nullptr, c);
    for (int blk = c.blk0; blk < c.blk1; ++blk) {
        M3_DCHECK(p, g.t0 == (int64_t)blk * p.TB && g.Tv >= 1 && g.Tv <= p.TB && g.t0 + g.Tv <= p.T);
        lds_barrier();  // previous block's readers of the LDS planes are done
        stage_scalars_x<Io>(rb, sm, p, c, g);
        const BlockGeo gn = block_geo(p, blk + 1);
        if constexpr (VEC) {
            if (blk + 1 < c.blk1) load_block<Io, kLoadXs>(rb, p, c, gn);  // x, dt, lambda: consumed
        }
        if constexpr (!VEC) stage_angles_table<Cfg>(sm, p, g);
        block_angle_totals<Cfg>(sm, p, g);
        stage_prologue<Io>(rb, sm, p, c, g, ct_unused, false);
        if (blk + 1 < c.blk1) load_block<Io, VEC ? kLoadBc : kLoadAll>(rb, p, c, gn);
        lds_barrier();
        const float cs_end = sm.cs[Cfg::ROWS - 1];
        carry_block<Cfg>(sm, sagg, __expf(cs_end));
        if constexpr (Cfg::MV) {
            if (blk + 1 < c.blk1) stage_raw_bc<Cfg>(rb, (uint16_t *)sm.raw, nullptr, c);
        }
        lsum += cs_end;
        if (tid < N2) sm.base[tid] += (double)sm.pend[tid];
        g = gn;
    }
    // segment aggregate -> workspace, in fragment order (one 16-byte store per tile and lane)
    const int wave = tid >> 6;
    const int64_t bs = c.bh * p.nsub + c.seg;
    M3_DCHECK(p, c.seg < p.nsub && p.Sagg && p.lseg && p.pseg && p.cseg);
    float *Sg = p.Sagg + ((c.bh * p.ncg + c.cg) * p.nsub + c.seg) * (int64_t)(NP * PP);
#pragma unroll
    for (int m = 0; m < Cfg::TPW; ++m) {
        int nt, pt;
        if (!state_tile<Cfg>(m, nt, pt)) continue;
        *(f32x4_t *)(Sg + ((size_t)(wave + 4 * m) * 64 + lane) * 4) = sagg[m];
    }
    if (c.cg != 0) return;  // the segment's decay and angle are the same for every column group
    if (tid == 0) p.lseg[bs] = lsum;
    lds_barrier();
    if (tid < NP / 2) {
        const double a = tid < N2 ? wrap_2pi(sm.base[tid]) : 0.0;
        const f32x2_t sc_ = sincos_acc((float)a);
        p.pseg[bs * p.np2 + tid] = (float)a;
        *(f32x2_t *)(p.cseg + (bs * p.np2 + tid) * 2) = f32x2_t{sc_[1], sc_[0]};
    }
}

// ============================================================ column-owned outputs
// (rank-1 bf16 path with 64 columns per workgroup)
//
// The G o L tiles of a block (t tile T >= s tile S, 16 x 16 each) are computed once, spread over
// the waves so that each does about the same work (a diagonal tile, with the full mask, costs
// more than a strictly causal one, whose decay factors), masked, with D on the diagonal (so
// that Y_intra includes D x), and written to the G o L planes [t][s] as bf16 hi / lo.  Tiles
// above the diagonal that share a 32-wide k step with causal ones ((0, 1) and (2, 3)) stay 0.
// Wave w then computes Y^T for its 16 columns p = 16w .. 16w + 15 and every row:
//     Y^T = diag-scaled (H^T C~^T) + X^T (G o L)^T
// H^T from the state columns the wave itself holds (fp16 with a per-wave power-of-two scale),
// C~^T and (G o L)^T from LDS; a result fragment holds 4 consecutive columns of one row, stored
// to y as 8 bytes.
// Tiles of wave w (nibble q; 15 = none): w0 (0,0) (3,3); w1 (1,1) (2,2); w2 (1,0) (2,0) (3,0);
// w3 (2,1) (3,1) (3,2).
__device__ __forceinline__ void gl_tile(int w, int q, int &T, int &S) {
    const unsigned tt_ = w == 0 ? 0xF30u : w == 1 ? 0xF21u : w == 2 ? 0x321u : 0x332u;
    const unsigned ss_ = w == 0 ? 0xF30u : w == 1 ? 0xF21u : w == 2 ? 0x000u : 0x211u;
    T = (int)((tt_ >> (4 * q)) & 15u);
    S = (int)((ss_ >> (4 * q)) & 15u);
}

// Gate input z in the column-owned epilogue's mapping: for each 16-row tile T, columns
// 16w + 4g .. 16w + 4g + 3 of row 16T + l16 (8 bytes).
struct RawZCol {
    u32x2_t w[4];
};
template <class Io>
__device__ __forceinline__ void load_z_col(RawZCol &rz, const ScanParams &p, const WgCtx &c, const BlockGeo &g) {
    using ET = typename Io::T;
    const int lane = threadIdx.x & 63, l16 = lane & 15, gq = lane >> 4;
    const int pc = row_tile() * 16 + 4 * gq;
    const ET *zb = (const ET *)c.zb + (int64_t)g.t0 * c.sz;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
        const int t = T * 16 + l16;
        u32x2_t v = {0u, 0u};
        if (t < g.Tv && pc < c.Pw) v = *(const u32x2_t *)(zb + (uint32_t)(t * c.sz + pc));
        rz.w[T] = v;
    }
}

// The zero tiles (0, 1) and (2, 3) of both G o L planes (written once per workgroup).
template <class Cfg, class Sm>
__device__ __forceinline__ void init_gl_zero_tiles(const Sm &sm) {
    const int tid = ltid();  // 256 threads: (plane, tile, row, 4-column group) -> 2 x 2 x 16 x 4
    const int pl = tid >> 7, tl = (tid >> 6) & 1, r = (tid >> 2) & 15, cg = tid & 3;
    const int T = tl ? 2 : 0, S = tl ? 3 : 1;
    uint16_t *gp = (uint16_t *)sm.gl + pl * Cfg::GL_PLANE;
    *(u32x2_t *)(gp + (T * 16 + r) * Cfg::RPP + S * 16 + 4 * cg) = u32x2_t{0u, 0u};
}

template <class Io, class Cfg, bool GATE, class Sm>
__device__ __forceinline__ void col_outputs(const Sm &sm, const ScanParams &p, const WgCtx &c, const BlockGeo &g,
                                            const f32x4_t (&hs)[Cfg::TPW], const RawZCol &rz) {
    using ET = typename Io::T;
    constexpr int KS = Cfg::KS, OPP = Cfg::OPP, RPP = Cfg::RPP;
    const int lane = threadIdx.x & 63, l16 = lane & 15, gq = lane >> 4;
    const int w = row_tile();
    const uint16_t *bt = (const uint16_t *)sm.bt, *ctp = (const uint16_t *)sm.ct;
    uint16_t *glh = (uint16_t *)sm.gl, *gll = glh + Cfg::GL_PLANE;
    const float Dh = p.D[c.h];
    // ---- this wave's G o L tiles
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        int T, S;
        gl_tile(w, q, T, S);
        if (T == 15) break;
        f32x4_t gv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const FragH a{*(const u32x4_t *)(bt + (S * 16 + l16) * OPP + kk * 32 + 8 * gq)};
            const FragH b{*(const u32x4_t *)(ctp + (T * 16 + l16) * OPP + kk * 32 + 8 * gq)};
            gv = mma(a, b, gv);
        }
        const int trow = T * 16 + l16, sb = S * 16 + 4 * gq;  // slot i: G[t = trow][s = sb + i]
        if (c.rowscale) gv *= *(const f32x4_t *)(sm.isr + sb) * sm.isr[Cfg::ROWS + trow];
        const float cs_t = sm.cs[trow];
        float mv[4];
        if (S < T) {
            // strictly causal tile: exp(cs_t - cs_ref) u_s
            const f32x4_t us = *(const f32x4_t *)(sm.u + sb);
            const float et = __expf(cs_t - sm.cs[S * 16 + 15]);
#pragma unroll
            for (int i = 0; i < 4; ++i) mv[i] = gv[i] * (et * us[i]);
        } else {
            const f32x4_t css = *(const f32x4_t *)(sm.cs + sb);
            const f32x4_t scs = *(const f32x4_t *)(sm.scale + sb);
            const float g_t = sm.gam[trow];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = sb + i;
                mv[i] = s < trow ? gv[i] * (__expf(cs_t - css[i]) * scs[i]) : (s == trow ? fmaf(gv[i], g_t, Dh) : 0.f);
            }
        }
        uint32_t h0, l0, h1, l1;
        split2(mv[0], mv[1], h0, l0);
        split2(mv[2], mv[3], h1, l1);
        const int off = trow * RPP + sb;
        *(u32x2_t *)(glh + off) = u32x2_t{h0, h1};
        *(u32x2_t *)(gll + off) = u32x2_t{l0, l1};
    }
    // the block's angle totals and their (cos, sin) for the carry, on the wave with three
    // strictly causal tiles (no per-element decays): it has slack before this barrier
    if (w == 2) block_angle_totals<Cfg>(sm, p, g, 2);
    lds_barrier();
    // ---- H^T of this wave's columns as fp16 A operands: k step mm covers state tiles 2mm, 2mm+1
    // (slot j < 4: n = 32mm + 4g + j; j >= 4: n = 32mm + 16 + 4g + j - 4)
    float hsc, hinv;
    {
        float m = 0.f;
#pragma unroll
        for (int k = 0; k < Cfg::TPW; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(hs[k][i]));
        pow2_scale<14>(wave_max_nonneg(m), hsc, hinv);
    }
    u32x4_t ha[KS];
#pragma unroll
    for (int mm = 0; mm < KS; ++mm)
        ha[mm] = u32x4_t{pack_f16(hs[2 * mm][0] * hsc, hs[2 * mm][1] * hsc), pack_f16(hs[2 * mm][2] * hsc, hs[2 * mm][3] * hsc),
                         pack_f16(hs[2 * mm + 1][0] * hsc, hs[2 * mm + 1][1] * hsc),
                         pack_f16(hs[2 * mm + 1][2] * hsc, hs[2 * mm + 1][3] * hsc)};
    // X^T of this wave's columns (exact bf16): p = 16w + l16, s = 32kk + 8g .. + 7
    u32x4_t xa[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) xa[kk] = *(const u32x4_t *)((const uint16_t *)sm.xt + xt_off<Cfg>(w * 16 + l16, kk * 32 + 8 * gq));
    const int pc = w * 16 + 4 * gq;
    ET *const yblk = (ET *)c.yb + g.t0 * c.sy;  // this block's first output row (row offsets fit 32 bits)
    // two row tiles at a time: every LDS operand of the pair is requested before its products
#pragma unroll
    for (int T0 = 0; T0 < 4; T0 += 2) {
        u32x4_t cb[2][KS];
        FragHL gb[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = (T0 + u) * 16 + l16;
#pragma unroll
            for (int mm = 0; mm < KS; ++mm) {
                const u32x2_t b0 = *(const u32x2_t *)(ctp + t * OPP + mm * 32 + 4 * gq);
                const u32x2_t b1 = *(const u32x2_t *)(ctp + t * OPP + mm * 32 + 16 + 4 * gq);
                cb[u][mm] = u32x4_t{b0[0], b0[1], b1[0], b1[1]};
            }
#pragma unroll
            for (int kk = 0; kk <= (T0 >> 1); ++kk) {
                gb[u][kk].hi = *(const u32x4_t *)(glh + t * RPP + kk * 32 + 8 * gq);
                gb[u][kk].lo = *(const u32x4_t *)(gll + t * RPP + kk * 32 + 8 * gq);
            }
        }
        f32x4_t acc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mm = 0; mm < KS; ++mm) acc[u] = mfma_h(ha[mm], cb[u][mm], acc[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = (T0 + u) * 16 + l16;
            float f = sm.ecs[t] * hinv;  // exp(cs_t) and the inverse scales of H and of the C~ row
            if (c.rowscale) f *= sm.isr[Cfg::ROWS + t];
            acc[u] *= f;
        }
#pragma unroll
        for (int kk = 0; kk <= (T0 >> 1); ++kk)
#pragma unroll
            for (int u = 0; u < 2; ++u) acc[u] = mma(xa[kk], gb[u][kk], acc[u]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int T = T0 + u, t = T * 16 + l16;
            // epilogue: the gate, one rounding, 4 consecutive columns of row t
            float yv[4] = {acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
            if constexpr (GATE) {
                const u32x2_t zw = rz.w[T];
                const float zv[4] = {__uint_as_float(zw[0] << 16), __uint_as_float(zw[0] & 0xffff0000u),
                                     __uint_as_float(zw[1] << 16), __uint_as_float(zw[1] & 0xffff0000u)};
#pragma unroll
                for (int i = 0; i < 4; ++i) yv[i] *= silu_f(zv[i]);
            }
            M3_DCHECK(p, !(t < g.Tv && pc < c.Pw) || (g.t0 + t < p.T && c.p0 + pc + 4 <= p.P));
            if (t < g.Tv && pc < c.Pw)
                *(u32x2_t *)(yblk + (uint32_t)(t * c.sy + pc)) = u32x2_t{pack_bf16(yv[0], yv[1]), pack_bf16(yv[2], yv[3])};
        }
    }
}

// ============================================================ output kernel
// With N above 64 the LDS planes allow one workgroup per compute unit (one wave per
// SIMD), so such variants may use the whole register file.
template <class Io, int NP, int PP, int MODE, bool GATE, bool PJ, bool HS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NP > 64 ? 1 : 2, NP > 64 ? 1 : 2))) void seg_output_kernel(ScanParams p) {
    using Cfg = SegCfg<Io, NP, PP, MODE, !GATE, PJ, HS>;
    constexpr bool VEC = Cfg::VEC;
    using ET = typename Io::T;
    using Frag = typename std::conditional<Cfg::BF, FragH, FragF>::type;
    constexpr int KS = Cfg::KS, PT = Cfg::PT, TPW = Cfg::TPW;
    constexpr int OPP = Cfg::OPP, RPP = Cfg::RPP;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const Smem<Cfg, true> sm(smem);
    const WgCtx c = make_ctx<Cfg>(p, p.nseg, p.bps);
    const int tid = ltid(), lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, gq = lane >> 4;
    const int N = p.N, P = p.P, N2 = N / 2;
    const int R = VEC ? 1 : c.R;
    const int64_t bh = c.bh;
    const bool want_final = (c.seg == p.nseg - 1) && (p.h1 != nullptr);

    // prefetch the first block while the incoming state is assembled
    stage_affine<Cfg>(sm, p, c);
    init_pad_pairs<Cfg>(sm, p);
    RawBlock<Cfg, true> rb;
    RawZ<Cfg> rz;
    RawZCol rzc;
    BlockGeo g = block_geo(p, c.blk0);
    // With a MIMO projection of z or y the epilogue reads z from memory itself (the y staging
    // area then holds fp32 per-rank outputs); otherwise z is prefetched into that area.
    const bool proj_o = Cfg::PJ && p.mo;
    const bool zpre = GATE && !(Cfg::PJ && (p.mz || p.mo));
    if constexpr (GATE) {
        if constexpr (Cfg::COL) load_z_col<Io>(rzc, p, c, g);
        else if (zpre) load_z<Io>(rz, p, c, g);
    }
    if constexpr (Cfg::COL) init_gl_zero_tiles<Cfg>(sm);
    load_block<Io>(rb, p, c, g);

    // ---- incoming state H (this wave's state fragments) and, for the final state, the
    // global angle at the segment's start: from the prefix kernel when it ran, otherwise
    // assembled here from the initial state and the earlier segments' aggregates (then one
    // state sub-segment per output segment)
    f32x4_t hs[TPW];
    if (p.Hin) {
        M3_DCHECK(p, c.seg < p.nseg);
        const float *Hg = p.Hin + ((bh * p.ncg + c.cg) * p.nseg + c.seg) * (int64_t)(NP * PP);
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            hs[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            int nt, pt;
            if (state_tile<Cfg>(m, nt, pt)) hs[m] = *(const f32x4_t *)(Hg + ((size_t)(wave + 4 * m) * 64 + lane) * 4);
        }
        if (want_final && tid < N2) {
            // global angle at this (last) segment's start: the initial angle plus every
            // state sub-segment's angle total
            double a = init_angle(p, bh, tid);
            constexpr int KB = 16;
            for (int j0 = 0; j0 < p.nsub; j0 += KB) {
                float v[KB];
#pragma unroll
                for (int k = 0; k < KB; ++k) v[k] = p.pseg[(bh * p.nsub + min(j0 + k, p.nsub - 1)) * p.np2 + tid];
#pragma unroll
                for (int k = 0; k < KB; ++k)
                    if (j0 + k < p.nsub) a += (double)v[k];
            }
            sm.base[tid] = a;
        }
    } else {
        {
            const float eta0 = (p.pB0 && p.px0) ? eta_first(p, c.b, c.h) : 0.f;
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
                hs[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                int nt, pt;
                if (!state_tile<Cfg>(m, nt, pt)) continue;
                const int pp = pt * 16 + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int nn = nt * 16 + 4 * gq + i;
                    float v = 0.f;
                    if (pp < c.Pw && nn < N) {
                        if (p.h0) v = p.h0[(bh * N + nn) * P + c.p0 + pp];
                        if (p.pB0 && p.px0) {
                            float acc = 0.f;
                            for (int r = 0; r < R; ++r)
                                acc += p.pB0[(bh * N + nn) * R + r] * p.px0[(bh * P + c.p0 + pp) * R + r];
                            v += eta0 * acc;
                        }
                    }
                    hs[m][i] = v;
                }
                if (!Cfg::HS && p.ang0) {
                    // rotate by -Theta_init
                    const int pr = (nt * 16 + 4 * gq) >> 1;
                    float s0 = 0.f, c0 = 1.f, s1 = 0.f, c1 = 1.f;
                    if (pr < p.nr) { const f32x2_t sc_ = sincos_acc((float)wrap_2pi((double)p.ang0[bh * p.nr + pr])); s0 = sc_[0]; c0 = sc_[1]; }
                    if (pr + 1 < p.nr) { const f32x2_t sc_ = sincos_acc((float)wrap_2pi((double)p.ang0[bh * p.nr + pr + 1])); s1 = sc_[0]; c1 = sc_[1]; }
                    rot_neg(hs[m], c0, s0, c1, s1);
                }
            }
            if (Cfg::HS && p.ang0) {
                // rotate by -Theta_init (half-split: rows n and n + N/2 of pair n)
#pragma unroll
                for (int m = 0; m < Cfg::HSM; ++m) {
                    int nt, pt;
                    state_tile<Cfg>(m, nt, pt);
                    const int n0 = nt * 16 + 4 * gq;
                    float cs[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float sn = 0.f, cn = 1.f;
                        if (n0 + i < p.nr) fast_sincos((float)wrap_2pi((double)p.ang0[bh * p.nr + n0 + i]), sn, cn);
                        cs[2 * i] = cn;
                        cs[2 * i + 1] = sn;
                    }
                    rot_neg_hs(hs[m], hs[m + Cfg::HSM], f32x4_t{cs[0], cs[1], cs[2], cs[3]},
                               f32x4_t{cs[4], cs[5], cs[6], cs[7]});
                }
            }
            // fold the earlier segments: H <- Rot(-Phi_s) (exp(l_s) H) + S_s (the aggregate is
            // already in its segment's end frame).  FB segments at a time: each wave loads its
            // tiles of all FB aggregates at once (slots past the last segment reload it and are
            // not applied), while the workgroup stages the FB segments' (cos, sin) per pair and
            // decays in LDS (the B~ plane, free until the first block's prologue), so that one
            // round trip to memory serves up to FB segments.
            constexpr int FB = TPW <= 2 ? 16 : TPW <= 4 ? 8 : 4;
            static_assert((FB * NP + FB) * sizeof(float) <= Cfg::L_BT, "fold tables exceed the B~ plane");
            const int64_t q = bh * p.ncg + c.cg;
            float *fcs = (float *)sm.bt;              // [FB][np2][2] (cos, sin)
            float *flg = fcs + FB * Cfg::NP;          // [FB] decay log
            for (int s0 = 0; s0 < c.seg; s0 += FB) {
                const int nk = min(FB, c.seg - s0);
                f32x4_t sv[FB][TPW];
#pragma unroll
                for (int k = 0; k < FB; ++k) {
                    const int s2 = min(s0 + k, c.seg - 1);
                    const float *Sg = p.Sagg + (q * p.nsub + s2) * (int64_t)(NP * PP);
#pragma unroll
                    for (int m = 0; m < TPW; ++m) {
                        int nt, pt;
                        if (!state_tile<Cfg>(m, nt, pt)) continue;
                        sv[k][m] = *(const f32x4_t *)(Sg + ((size_t)(wave + 4 * m) * 64 + lane) * 4);
                    }
                }
                {
                    // the nk segments' (cos, sin) tables are contiguous: [nk][np2][2] floats
                    const float *cb = p.cseg + (bh * p.nsub + s0) * (int64_t)p.np2 * 2;
                    const int nv = nk * p.np2 / 2;  // float4s
                    M3_DCHECK(p, p.np2 <= Cfg::NP / 2 && nv * 4 <= FB * Cfg::NP);
                    for (int v = tid; v < nv; v += 256) *(f32x4_t *)(fcs + 4 * v) = *(const f32x4_t *)(cb + 4 * v);
                    if (tid < nk) flg[tid] = p.lseg[bh * p.nsub + s0 + tid];
                }
                lds_barrier();
#pragma unroll
                for (int k = 0; k < FB; ++k) {
                    if (k >= nk) break;
                    const float dec = __expf(flg[k]);
                    const float *ck = fcs + k * p.np2 * 2;
                    if constexpr (Cfg::HS) {
#pragma unroll
                        for (int m = 0; m < Cfg::HSM; ++m) {
                            int nt, pt;
                            state_tile<Cfg>(m, nt, pt);
                            // (cos, sin) of pairs n0 .. n0 + 3 (tile m < HSM) pair rows m and m + HSM
                            const float *cp = ck + (nt * 16 + 4 * gq) * 2;
                            f32x4_t a = dec * hs[m], b = dec * hs[m + Cfg::HSM];
                            rot_neg_hs(a, b, *(const f32x4_t *)cp, *(const f32x4_t *)(cp + 4));
                            hs[m] = a + sv[k][m];
                            hs[m + Cfg::HSM] = b + sv[k][m + Cfg::HSM];
                        }
                    } else {
#pragma unroll
                        for (int m = 0; m < TPW; ++m) {
                            int nt, pt;
                            if (!state_tile<Cfg>(m, nt, pt)) continue;
                            // (cos, sin) of pairs nt*8 + 2*gq and the next one
                            const f32x4_t cs4 = *(const f32x4_t *)(ck + (nt * 8 + 2 * gq) * 2);
                            f32x4_t a = dec * hs[m];
                            rot_neg(a, cs4[0], cs4[1], cs4[2], cs4[3]);
                            hs[m] = a + sv[k][m];
                        }
                    }
                }
                if (s0 + FB < c.seg) lds_barrier();  // the next round rewrites the tables
            }
            if (tid < N2) {
                double a = init_angle(p, bh, tid);
                for (int s0 = 0; s0 < c.seg; s0 += FB) {
                    float v[FB];
#pragma unroll
                    for (int k = 0; k < FB; ++k) v[k] = p.pseg[(bh * p.nsub + min(s0 + k, c.seg - 1)) * p.np2 + tid];
#pragma unroll
                    for (int k = 0; k < FB; ++k)
                        if (s0 + k < c.seg) a += (double)v[k];
                }
                sm.base[tid] = a;
            }
        }
    }

    if constexpr (!Cfg::COL) publish_hmax<Cfg>(sm, hs);  // the incoming state's magnitude, for its fp16 scale
    Frag ct[KS];
    for (int blk = c.blk0; blk < c.blk1; ++blk) {
        M3_DCHECK(p, g.t0 == (int64_t)blk * p.TB && g.Tv >= 1 && g.Tv <= p.TB && g.t0 + g.Tv <= p.T);
        lds_barrier();  // every wave is done with the previous block's LDS planes
        float inv_hs = 1.f;
        if constexpr (!Cfg::COL) {
            if (zpre) stage_z<Cfg>(rz, sm, c);  // read by the epilogue after two more barriers
            inv_hs = write_ht<Cfg>(sm, hs);  // the state entering this block (read after two more barriers)
        }
        if constexpr (Cfg::MV) stage_raw_bc<Cfg>(rb, (uint16_t *)sm.bt, (uint16_t *)sm.bt + Cfg::BT_PLANE, c);
        stage_scalars_x<Io>(rb, sm, p, c, g);
        const BlockGeo gn = block_geo(p, blk + 1);
        if constexpr (VEC) {
            // the next block's x, dt, lambda as soon as this block's are staged
            if (blk + 1 < c.blk1) load_block<Io, kLoadXs>(rb, p, c, gn);
        }
        if constexpr (!VEC) stage_angles_table<Cfg>(sm, p, g);
        // (column-owned outputs: on wave 2, which has slack before col_outputs' barrier)
        if constexpr (!Cfg::COL) block_angle_totals<Cfg>(sm, p, g);
        stage_prologue<Io>(rb, sm, p, c, g, ct, want_final && c.cg == 0 && blk == c.blk1 - 1);
        if constexpr (VEC) {
            // and its B, C, theta once the prologue has consumed this block's
            if (blk + 1 < c.blk1) load_block<Io, kLoadBc>(rb, p, c, gn);
        }
        lds_barrier();

        if constexpr (Cfg::COL) {
            col_outputs<Io, Cfg, GATE>(sm, p, c, g, hs, rzc);
            if constexpr (GATE) {
                if (blk + 1 < c.blk1) load_z_col<Io>(rzc, p, c, gn);
            }
        } else {
        // ---- outputs for this wave's 16 rows
        const int tt = row_tile();
        const int row0 = tt * 16 + 4 * gq;  // result rows row0 .. row0 + 3 of this lane
        f32x4_t yacc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) yacc[pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // Y_inter = C~ H first, then scaled by exp(cs_t) per row; Y_intra accumulates on top
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int ho = (pt * 16 + l16) * OPP + kk * 32 + 8 * gq;
                if constexpr (Cfg::F16) {
                    const FragH hf{*(const u32x4_t *)((const uint16_t *)sm.ht + ho)};
                    yacc[pt] = mma(ct[kk], hf, yacc[pt]);
                } else {
                    FragF hf;
                    const f32x4_t v0 = *(const f32x4_t *)((const float *)sm.ht + ho);
                    const f32x4_t v1 = *(const f32x4_t *)((const float *)sm.ht + ho + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) { hf.v[j] = v0[j]; hf.v[j + 4] = v1[j]; }
                    yacc[pt] = mma(ct[kk], hf, yacc[pt]);
                }
            }
        }
        {
            // exp(cs_t), times the inverse scales of H and of the C~ rows (fp16 operands)
            f32x4_t ecs4;
            if constexpr (VEC) {
                ecs4 = *(const f32x4_t *)(sm.ecs + row0);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) ecs4[i] = sm.ecs[tok_of(row0 + i, c)];
            }
            ecs4 *= inv_hs;
            if (c.rowscale) ecs4 *= *(const f32x4_t *)(sm.isr + Cfg::ROWS + row0);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) yacc[pt] *= ecs4;
        }
        const int trow = tt * 16 + l16;  // this lane's t-row in the G^T fragments
        const int ttok = VEC ? trow : tok_of(trow, c);
        const float cs_t = sm.cs[ttok], g_t = sm.gam[ttok];
        const float isc_t = c.rowscale ? sm.isr[Cfg::ROWS + trow] : 1.f;  // inverse scale of C~ row t
        int smax = tt;
        if constexpr (!VEC) {
            // with R not dividing 16 the rows of the tile's last token may spill into the next tile
            smax = ((tok_of(tt * 16 + 15, c)) * R + R - 1) >> 4;
            if (smax > Cfg::ROWS / 16 - 1) smax = Cfg::ROWS / 16 - 1;
        }
        for (int sp = 0; sp <= smax / 2; ++sp) {
            const int st0 = 2 * sp, st1 = 2 * sp + 1;
            const bool has1 = st1 <= smax;
            f32x4_t g0 = {0.f, 0.f, 0.f, 0.f}, g1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const int o0 = (st0 * 16 + l16) * OPP + kk * 32 + 8 * gq;
                const int o1 = (st1 * 16 + l16) * OPP + kk * 32 + 8 * gq;
                if constexpr (Cfg::F16) {
                    const uint16_t *bt = (const uint16_t *)sm.bt;
                    g0 = mma(FragH{*(const u32x4_t *)(bt + o0)}, ct[kk], g0);
                    if (has1) g1 = mma(FragH{*(const u32x4_t *)(bt + o1)}, ct[kk], g1);
                } else {
                    const float *bt = (const float *)sm.bt;
                    FragF a0;
                    const f32x4_t u0 = *(const f32x4_t *)(bt + o0), u1 = *(const f32x4_t *)(bt + o0 + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) { a0.v[j] = u0[j]; a0.v[j + 4] = u1[j]; }
                    g0 = mma(a0, ct[kk], g0);
                    if (has1) {
                        FragF a1;
                        const f32x4_t v0 = *(const f32x4_t *)(bt + o1), v1 = *(const f32x4_t *)(bt + o1 + 4);
#pragma unroll
                        for (int j = 0; j < 4; ++j) { a1.v[j] = v0[j]; a1.v[j + 4] = v1[j]; }
                        g1 = mma(a1, ct[kk], g1);
                    }
                }
            }
            // mask: slot i of g0 is G[t = trow][s = st0*16 + 4g + i]
            float mv[8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int st = half ? st1 : st0;
                const int sb = st * 16 + 4 * gq;
                f32x4_t gv = half ? g1 : g0;
                if (half && !has1) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) mv[4 + i] = 0.f;
                    continue;
                }
                if (c.rowscale) gv *= *(const f32x4_t *)(sm.isr + sb) * isc_t;  // undo the fp16 row scales
                if constexpr (VEC) {
                    if (st < tt) {
                        // a strictly earlier s tile: the factored decay exp(cs_t - cs_ref) u_s
                        const f32x4_t us = *(const f32x4_t *)(sm.u + sb);
                        const float et = __expf(cs_t - sm.cs[st * 16 + 15]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) mv[half * 4 + i] = gv[i] * (et * us[i]);
                        continue;
                    }
                    const f32x4_t css = *(const f32x4_t *)(sm.cs + sb);
                    const f32x4_t scs = *(const f32x4_t *)(sm.scale + sb);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s = sb + i;
                        const float L = s < trow ? __expf(cs_t - css[i]) * scs[i] : (s == trow ? g_t : 0.f);
                        mv[half * 4 + i] = gv[i] * L;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int stok = tok_of(sb + i, c);
                        const float L = stok < ttok ? __expf(cs_t - sm.cs[stok]) * sm.scale[stok]
                                                    : (stok == ttok ? g_t : 0.f);
                        mv[half * 4 + i] = gv[i] * L;
                    }
                }
            }
            // G o L as the A operand of Y_intra: bf16 hi/lo (X is exact bf16) or fp32
            typename std::conditional<Cfg::BF, FragHL, FragF>::type mf;
            if constexpr (Cfg::BF) mf = make_hl(mv);
            else mf = make_f(mv);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int xo0 = xt_off<Cfg>(pt * 16 + l16, st0 * 16 + 4 * gq);
                const int xo1 = xt_off<Cfg>(pt * 16 + l16, st1 * 16 + 4 * gq);
                if constexpr (Cfg::BF) {
                    const u32x2_t x0 = *(const u32x2_t *)((const uint16_t *)sm.xt + xo0);
                    u32x2_t x1 = {0u, 0u};
                    if (has1) x1 = *(const u32x2_t *)((const uint16_t *)sm.xt + xo1);
                    const u32x4_t xb = {x0[0], x0[1], x1[0], x1[1]};
                    yacc[pt] = mma(mf, xb, yacc[pt]);
                } else {
                    FragF xb;
                    const f32x4_t x0 = *(const f32x4_t *)((const float *)sm.xt + xo0);
                    f32x4_t x1 = {0.f, 0.f, 0.f, 0.f};
                    if (has1) x1 = *(const f32x4_t *)((const float *)sm.xt + xo1);
#pragma unroll
                    for (int j = 0; j < 4; ++j) { xb.v[j] = x0[j]; xb.v[j + 4] = x1[j]; }
                    yacc[pt] = mma(mf, xb, yacc[pt]);
                }
            }
        }

        // ---- epilogue: y = exp(cs_t) Y_inter + Y_intra + D x, times silu(z) with the gate,
        // rounded once -> staging (own rows)
        {
            ET *ys = (ET *)sm.ys;
            const float Dh = p.D[c.h];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int pc = pt * 16 + l16;
                float xv[4];
                if constexpr (Cfg::BF) {
                    const u32x2_t x2 = *(const u32x2_t *)((const uint16_t *)sm.xt + xt_off<Cfg>(pc, row0));
                    xv[0] = __uint_as_float(x2[0] << 16);
                    xv[1] = __uint_as_float(x2[0] & 0xffff0000u);
                    xv[2] = __uint_as_float(x2[1] << 16);
                    xv[3] = __uint_as_float(x2[1] & 0xffff0000u);
                } else {
                    const f32x4_t x4 = *(const f32x4_t *)((const float *)sm.xt + xt_off<Cfg>(pc, row0));
#pragma unroll
                    for (int i = 0; i < 4; ++i) xv[i] = x4[i];
                }
                float yv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) yv[i] = yacc[pt][i] + Dh * xv[i];
                if (GATE && !zpre) {
                    // z read from memory: rank-free and expanded by mimo_z[h, r, :], or per rank
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tk = tok_of(row0 + i, c), r = row0 + i - tk * R;
                        float zv = 0.f;
                        if (tk < g.Tv && pc < c.Pw) {
                            const ET *zr = (const ET *)c.zb + (int64_t)(g.t0 + tk) * c.sz;
                            zv = p.mz ? Io::ld(zr + pc) * p.mz[((int64_t)c.h * R + r) * p.P + c.p0 + pc]
                                      : Io::ld(zr + (int64_t)pc * R + r);
                        }
                        yv[i] *= silu_f(zv);
                    }
                } else if constexpr (GATE) {
                    // z of these outputs, staged at the positions their y values take
                    float zv[4];
                    if constexpr (Cfg::MV) {
                        u32x2_t zw;
                        if (R == 2) {
                            const int tk = row0 >> 1;
                            zw[0] = *(const uint32_t *)(ys + (tk * PP + pc) * 2);
                            zw[1] = *(const uint32_t *)(ys + ((tk + 1) * PP + pc) * 2);
                        } else {
                            const int tk = tok_of(row0, c), r0 = row0 - tk * R;
                            zw = *(const u32x2_t *)(ys + (tk * PP + pc) * R + r0);
                        }
                        zv[0] = __uint_as_float(zw[0] << 16);
                        zv[1] = __uint_as_float(zw[0] & 0xffff0000u);
                        zv[2] = __uint_as_float(zw[1] << 16);
                        zv[3] = __uint_as_float(zw[1] & 0xffff0000u);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) zv[i] = Io::ld(ys + ys_off<Cfg>(row0 + i, pc));
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) yv[i] *= silu_f(zv[i]);
                }
                if (proj_o) {
                    // per-rank outputs in fp32, [row][p], for the rank contraction below
#pragma unroll
                    for (int i = 0; i < 4; ++i) ((float *)sm.ys)[(row0 + i) * PP + pc] = yv[i];
                } else if constexpr (Cfg::MV) {
                    // staged in the global order [token][p][rank]
                    const uint32_t w01 = pack_bf16(yv[0], yv[1]), w23 = pack_bf16(yv[2], yv[3]);
                    if (R == 2) {
                        const int tk = row0 >> 1;
                        *(uint32_t *)(ys + (tk * PP + pc) * 2) = w01;
                        *(uint32_t *)(ys + ((tk + 1) * PP + pc) * 2) = w23;
                    } else {
                        const int tk = tok_of(row0, c), r0 = row0 - tk * R;
                        *(u32x2_t *)(ys + (tk * PP + pc) * R + r0) = u32x2_t{w01, w23};
                    }
                } else if constexpr (Cfg::BF) {
                    const uint32_t w01 = pack_bf16(yv[0], yv[1]), w23 = pack_bf16(yv[2], yv[3]);
                    ys[ys_off<Cfg>(row0 + 0, pc)] = (uint16_t)(w01 & 0xffffu);
                    ys[ys_off<Cfg>(row0 + 1, pc)] = (uint16_t)(w01 >> 16);
                    ys[ys_off<Cfg>(row0 + 2, pc)] = (uint16_t)(w23 & 0xffffu);
                    ys[ys_off<Cfg>(row0 + 3, pc)] = (uint16_t)(w23 >> 16);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) ys[ys_off<Cfg>(row0 + i, pc)] = yv[i];
                }
            }
        }
        // the next block's gate input (and, on the element and interleaved-rank paths, its
        // raw inputs), issued once this block's outputs are staged (they overlap the stores
        // and the carry)
        if (blk + 1 < c.blk1) {
            if (zpre) load_z<Io>(rz, p, c, gn);
            if constexpr (!VEC) load_block<Io>(rb, p, c, gn);
        }
        // ---- y: this wave's rows, staged in its own part of the staging area (LDS
        // operations of one wave complete in order), stored as 16-byte vectors
        if (proj_o) {
            // y[t, q] = sum_r mimo_o[h, r, q] y_r[t, q]: a token's ranks may lie in the rows
            // of two waves, so the whole block's staging is read after a barrier
            lds_barrier();
            const float *ysf = (const float *)sm.ys;
            const float *moh = p.mo + (int64_t)c.h * R * p.P + c.p0;
            for (int e = tid; e < g.Tv * PP; e += 256) {
                const int tk = e / PP, q = e - tk * PP;
                if (q >= c.Pw) continue;
                float acc = 0.f;
                for (int r = 0; r < R; ++r) acc += moh[(int64_t)r * p.P + q] * ysf[(tk * R + r) * PP + q];
                M3_DCHECK(p, g.t0 + tk < p.T && c.p0 + q < p.P);
                Io::st((ET *)c.yb + (g.t0 + tk) * c.sy + q, acc);
            }
        } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        {
            const ET *ys = (const ET *)sm.ys;
            const int Rv = g.Tv * R;
            if constexpr (Cfg::MV) {
                const int yvpt = (PP * R) >> 3;
                const float iy = 1.f / (float)yvpt;
                const int tk0 = (tt * 16) / R;
#pragma unroll
                for (int m = 0; m < 16 * PP / 8 / 64; ++m) {
                    const int e = lane + 64 * m;
                    const int tk = tk0 + (int)(((float)e + 0.5f) * iy), o = e - (tk - tk0) * yvpt;
                    M3_DCHECK(p, !(tk < g.Tv && o * 8 < c.Pw * R) || (g.t0 + tk < p.T && c.p0 * R + o * 8 + 8 <= p.P * R));
                    if (tk < g.Tv && o * 8 < c.Pw * R)
                        *(u32x4_t *)((ET *)c.yb + (g.t0 + tk) * c.sy + o * 8) = *(const u32x4_t *)(ys + tk * PP * R + o * 8);
                }
            } else if constexpr (VEC) {
#pragma unroll
                for (int m = 0; m < 16 * PP / Cfg::XW / 64; ++m) {
                    const int e = lane + 64 * m;
                    const int yr = tt * 16 + e / (PP / Cfg::XW), pc = (e % (PP / Cfg::XW)) * Cfg::XW;
                    M3_DCHECK(p, !(yr < Rv && pc < c.Pw) || (g.t0 + yr < p.T && c.p0 + pc + Cfg::XW <= p.P));
                    if (yr < Rv && pc < c.Pw)
                        *(u32x4_t *)((ET *)c.yb + (g.t0 + yr) * c.sy + pc) = *(const u32x4_t *)(ys + ys_off<Cfg>(yr, pc));
                }
            } else {
                for (int e = lane; e < 16 * PP; e += 64) {
                    const int yr = tt * 16 + e / PP, pc = e - (e / PP) * PP;
                    if (yr >= Rv || pc >= c.Pw) continue;
                    const int tok = tok_of(yr, c), r = yr - tok * R;
                    M3_DCHECK(p, g.t0 + tok < p.T && r >= 0 && r < R && c.p0 + pc < p.P);
                    ((ET *)c.yb)[(g.t0 + tok) * c.sy + (int64_t)pc * R + r] = ys[ys_off<Cfg>(yr, pc)];
                }
            }
        }
        }
        }  // row-owned outputs
        // ---- carry to the next block (H^T is rewritten after the next top barrier)
        const float cs_end = sm.cs[Cfg::ROWS - 1];
        carry_block<Cfg>(sm, hs, __expf(cs_end));
        if constexpr (!Cfg::COL) publish_hmax<Cfg>(sm, hs);
        // running angle at the next block's start (the last block's start angle is kept
        // for the carried B~ below)
        if (tid < N2 && blk + 1 < c.blk1) sm.base[tid] += (double)sm.pend[tid];
        g = gn;
    }
    if (want_final) {
        // The last block's B~ (B~ planes), x (X^T plane) and angle total are still in LDS.
        const BlockGeo gl = block_geo(p, c.blk1 - 1);
        lds_barrier();
        {
            // carried x of the last token
            const int lrow0 = (gl.Tv - 1) * R;
            for (int e = tid; e < c.Pw * R; e += 256) {
                const int pc = e / R, r = e - pc * R;
                float xv;
                if constexpr (Cfg::BF) xv = bf2f(((const uint16_t *)sm.xt)[xt_off<Cfg>(pc, lrow0 + r)]);
                else xv = ((const float *)sm.xt)[xt_off<Cfg>(pc, lrow0 + r)];
                M3_DCHECK(p, c.p0 + pc < P && lrow0 + r < Cfg::ROWS);
                p.px1[(bh * P + c.p0 + pc) * R + r] = xv;
            }
        }
        lds_barrier();  // every read of the last block's start angle is done
        if (tid < N2) sm.base[tid] += (double)sm.pend[tid];
        lds_barrier();  // final base angles visible
        // final state in the global frame: Rot(Theta_final) H
        f32x4_t hf[TPW];
        if constexpr (Cfg::HS) {
#pragma unroll
            for (int m = 0; m < Cfg::HSM; ++m) {
                int nt, pt;
                state_tile<Cfg>(m, nt, pt);
                const int n0 = nt * 16 + 4 * gq;
                float cs[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x2_t sc_ = sincos_acc((float)wrap_2pi(sm.base[n0 + i]));
                    cs[2 * i] = sc_[1];
                    cs[2 * i + 1] = -sc_[0];  // rotation by +Theta
                }
                hf[m] = hs[m];
                hf[m + Cfg::HSM] = hs[m + Cfg::HSM];
                rot_neg_hs(hf[m], hf[m + Cfg::HSM], f32x4_t{cs[0], cs[1], cs[2], cs[3]}, f32x4_t{cs[4], cs[5], cs[6], cs[7]});
            }
        }
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            int nt, pt;
            if (!state_tile<Cfg>(m, nt, pt)) continue;
            const int pp = pt * 16 + l16;
            f32x4_t a;
            if constexpr (Cfg::HS) {
                a = hf[m];
            } else {
                const int pr = (nt * 16 + 4 * gq) >> 1;
                float s0 = 0.f, c0 = 1.f, s1 = 0.f, c1 = 1.f;
                if (pr < N2) { const f32x2_t sc_ = sincos_acc((float)wrap_2pi(sm.base[pr])); s0 = sc_[0]; c0 = sc_[1]; }
                if (pr + 1 < N2) { const f32x2_t sc_ = sincos_acc((float)wrap_2pi(sm.base[pr + 1])); s1 = sc_[0]; c1 = sc_[1]; }
                a = hs[m];
                rot_neg(a, c0, -s0, c1, -s1);  // rotation by +Theta
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int nn = nt * 16 + 4 * gq + i;
                if (pp < c.Pw && nn < N) p.h1[(bh * N + nn) * P + c.p0 + pp] = a[i];
            }
        }
        if (c.cg == 0 && tid < p.nr) p.ang1[bh * p.nr + tid] = (float)wrap_2pi(sm.base[tid]);
    }
}

#ifdef M3_WITH_PREFIX_KERNEL
// ============================================================ prefix kernel
// Incoming state of every output segment: the initial state (h + eta_{-1} prev_B prev_x^T,
// rotated by -Theta_init into the frame of block 0) folded through the state sub-segments,
//     H <- Rot(-Phi_sub) (exp(l_sub) H) + S_sub,
// written at each output segment's start.  One thread per (sequence and column group,
// fragment float4 of the state); the sub-segment aggregates are loaded 16 at a time.
__global__ __launch_bounds__(256) void seg_prefix_kernel(ScanParams p) {
    const int NP = 2 * p.np2, PP = p.pp, PT = PP / 16;
    const int per_q = NP * PP / 4;
    const int nwg_q = (per_q + 255) / 256;
    const int64_t q = blockIdx.x / nwg_q;
    const int idx = (int)(blockIdx.x - q * nwg_q) * 256 + (int)threadIdx.x;
    const int64_t bh = q / p.ncg;
    const int cg = (int)(q - bh * p.ncg);
    const int64_t b = bh / p.H;
    const int h = (int)(bh - b * p.H);
    const int N = p.N, P = p.P, N2 = N / 2, R = p.R;
    const int p0 = cg * PP, Pw = min(PP, P - p0);
    const int kps = p.bps / p.sbps;  // state sub-segments per output segment
    M3_DCHECK(p, bh < p.B * p.H && cg < p.ncg && Pw >= 1 && p.Hin && kps * p.sbps == p.bps);
    if (idx < per_q) {
        const int e = idx >> 6, lane = idx & 63;
        const int nt = e / PT, pt = e - nt * PT, gq = lane >> 4, l16 = lane & 15;
        const int pp = pt * 16 + l16;
        f32x4_t H = {0.f, 0.f, 0.f, 0.f};
        if (p.h0 || (p.pB0 && p.px0)) {
            const float eta0 = (p.pB0 && p.px0) ? eta_first(p, b, h) : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int nn = nt * 16 + 4 * gq + i;
                float v = 0.f;
                if (pp < Pw && nn < N) {
                    if (p.h0) v = p.h0[(bh * N + nn) * P + p0 + pp];
                    if (p.pB0 && p.px0) {
                        float acc = 0.f;
                        for (int r = 0; r < R; ++r)
                            acc += p.pB0[(bh * N + nn) * R + r] * p.px0[(bh * P + p0 + pp) * R + r];
                        v += eta0 * acc;
                    }
                }
                H[i] = v;
            }
        }
        if (p.ang0) {
            // rotate by -Theta_init
            const int pr = (nt * 16 + 4 * gq) >> 1;
            float s0 = 0.f, c0 = 1.f, s1 = 0.f, c1 = 1.f;
            if (pr < p.nr) { const f32x2_t sc_ = sincos_acc((float)wrap_2pi((double)p.ang0[bh * p.nr + pr])); s0 = sc_[0]; c0 = sc_[1]; }
            if (pr + 1 < p.nr) { const f32x2_t sc_ = sincos_acc((float)wrap_2pi((double)p.ang0[bh * p.nr + pr + 1])); s1 = sc_[0]; c1 = sc_[1]; }
            rot_neg(H, c0, s0, c1, s1);
        }
        float *Ho = p.Hin + q * p.nseg * (int64_t)(NP * PP) + (size_t)idx * 4;
        *(f32x4_t *)Ho = H;
        constexpr int KB = 16;
        for (int j0 = 0; j0 < p.nsub; j0 += KB) {
            f32x4_t sv[KB], cs[KB];
            float lg[KB];
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int j = min(j0 + k, p.nsub - 1);
                const int64_t bs = bh * p.nsub + j;
                lg[k] = p.lseg[bs];
                sv[k] = *(const f32x4_t *)(p.Sagg + (q * p.nsub + j) * (int64_t)(NP * PP) + (size_t)idx * 4);
                cs[k] = *(const f32x4_t *)(p.cseg + (bs * p.np2 + nt * 8 + 2 * gq) * 2);
            }
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int j = j0 + k;
                if (j >= p.nsub) break;
                f32x4_t a = __expf(lg[k]) * H;
                rot_neg(a, cs[k][0], cs[k][1], cs[k][2], cs[k][3]);
                H = a + sv[k];
                if ((j + 1) % kps == 0) *(f32x4_t *)(Ho + (int64_t)((j + 1) / kps) * (NP * PP)) = H;
            }
        }
    }
}
#endif  // M3_WITH_PREFIX_KERNEL

// ---------------------------------------------------------------- launch helpers
template <class K>
static hipError_t set_lds(K kern, size_t bytes) {
    if (bytes > 65536)
        return hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    return hipSuccess;
}

template <class Io, int NP, int PP, int MODE, bool PJ, bool HS = false>
static hipError_t launch_seg_pj(bool output, const ScanParams &p, hipStream_t st) {
    using Cfg = SegCfg<Io, NP, PP, MODE, true, PJ, HS>;
    if (output) {
        // variant with the silu(z) output gate when z is given
        auto kern = p.z ? seg_output_kernel<Io, NP, PP, MODE, true, PJ, HS> : seg_output_kernel<Io, NP, PP, MODE, false, PJ, HS>;
        hipError_t e = set_lds(kern, Cfg::OUTPUT_BYTES);
        if (e != hipSuccess) return e;
        const int64_t nwg = p.B * p.H * (int64_t)p.ncg * p.nseg;
        hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(256), Cfg::OUTPUT_BYTES, st, p);
    } else {
        auto kern = seg_state_kernel<Io, NP, PP, MODE, PJ, HS>;
        hipError_t e = set_lds(kern, Cfg::STATE_BYTES);
        if (e != hipSuccess) return e;
        const int64_t nwg = p.B * p.H * (int64_t)p.ncg * p.nsub;
        if (nwg <= 0) return hipSuccess;
        hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(256), Cfg::STATE_BYTES, st, p);
    }
    return hipGetLastError();
}

// the projection variant when the call has MIMO projections (never on the rank-1 16-byte path)
// the half-split variant (rank-1 16-byte path with N = NP >= 64 only)
template <class Io, int NP, int PP, int MODE>
static hipError_t launch_seg_t(bool output, const TileShape &ts, const ScanParams &p, hipStream_t st) {
    if constexpr (MODE != kModeVec) {
        if (ts.hs) return hipErrorInvalidValue;
        if (ts.pj) return launch_seg_pj<Io, NP, PP, MODE, true>(output, p, st);
    } else {
        if (ts.pj) return hipErrorInvalidValue;
        if (ts.hs) {
            if constexpr (NP >= 64) return launch_seg_pj<Io, NP, PP, MODE, false, true>(output, p, st);
            else return hipErrorInvalidValue;
        }
    }
    return launch_seg_pj<Io, NP, PP, MODE, false>(output, p, st);
}
template <class Io, int NP, int PP, int MODE>
static size_t seg_bytes_t(bool output, const TileShape &ts) {
    using Cfg = SegCfg<Io, NP, PP, MODE>;
    using CfgP = SegCfg<Io, NP, PP, MODE, true, MODE != kModeVec>;
    if (ts.pj) return output ? CfgP::OUTPUT_BYTES : CfgP::STATE_BYTES;
    return output ? Cfg::OUTPUT_BYTES : Cfg::STATE_BYTES;
}

#define M3_SHAPES(X, Io, MODE) \
    X(Io, 32, 32, MODE) X(Io, 32, 64, MODE) X(Io, 64, 32, MODE) X(Io, 64, 64, MODE) X(Io, 128, 32, MODE) X(Io, 128, 64, MODE)

// Instantiate the launcher and LDS query of one (io type, load path) pair.
#define M3_DEFINE_VARIANT(NAME, Io, MODE)                                                              \
    hipError_t NAME##_launch(bool output, const TileShape &ts, const ScanParams &p, hipStream_t st) {  \
        M3_SHAPES(M3_LAUNCH_CASE, Io, MODE)                                                           \
        return hipErrorInvalidValue;                                                                  \
    }                                                                                                 \
    size_t NAME##_bytes(bool output, const TileShape &ts) {                                           \
        M3_SHAPES(M3_BYTES_CASE, Io, MODE)                                                            \
        return 0;                                                                                     \
    }
#define M3_LAUNCH_CASE(IoT, NPV, PPV, V) \
    if (ts.np == NPV && ts.pp == PPV) return launch_seg_t<IoT, NPV, PPV, V>(output, ts, p, st);
#define M3_BYTES_CASE(IoT, NPV, PPV, V) \
    if (ts.np == NPV && ts.pp == PPV) return seg_bytes_t<IoT, NPV, PPV, V>(output, ts);

}  // namespace m3
