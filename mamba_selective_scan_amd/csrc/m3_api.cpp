// m3_api.cpp -- the C ABI of libmamba3: argument checks, workspace layout and
// kernel dispatch.  Every check happens on the host before the first launch;
// nothing here allocates or synchronises.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/libmamba3.h"
#include "m3_internal.hpp"

namespace {

using m3::ScanParams;
using m3::StepParams;
using m3::TileShape;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------- debug builds
// With -DM3_DEBUG every kernel gets the device address of two words per GPU that its failed
// checks update (count, largest failing source line); m3_debug_checks reads and clears them.
#ifdef M3_DEBUG
static __device__ unsigned int dbg_words[2];
std::mutex g_dbg_mu;
unsigned int *g_dbg_ptr[64];
unsigned int *debug_words() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(g_dbg_mu);
    if (!g_dbg_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_words)) != hipSuccess) return nullptr;
        g_dbg_ptr[dev] = static_cast<unsigned int *>(p);
    }
    return g_dbg_ptr[dev];
}
#else
unsigned int *debug_words() { return nullptr; }
#endif

static_assert(M3_FLAG_BCNORM == m3::kFlagNorm && M3_FLAG_PARTIAL_ROPE == m3::kFlagPartialRope &&
                  M3_FLAG_A_PER_TOKEN == m3::kFlagAPerToken && M3_FLAG_DT_SOFTPLUS == m3::kFlagDtSoftplus &&
                  M3_FLAG_LAM_SIGMOID == m3::kFlagLamSigmoid && M3_FLAG_HALF_SPLIT == m3::kFlagHalfSplit,
              "flag values of the C ABI and the kernels differ");
constexpr uint32_t kAllFlags = M3_FLAG_BCNORM | M3_FLAG_PARTIAL_ROPE | M3_FLAG_A_PER_TOKEN | M3_FLAG_DT_SOFTPLUS |
                               M3_FLAG_LAM_SIGMOID | M3_FLAG_HALF_SPLIT;

// Rotated pairs: rope_pairs with M3_FLAG_PARTIAL_ROPE, otherwise all N/2.
int rotated_pairs(const m3_shape *s) {
    return (s->flags & M3_FLAG_PARTIAL_ROPE) ? s->rope_pairs : s->dstate / 2;
}

int pow2_at_least(int v, int lo) {
    int r = lo;
    while (r < v) r <<= 1;
    return r;
}

// Shape checks common to the scans and the step.  Returns M3_OK or an error.
m3_status check_shape(const m3_shape *s, bool step) {
    if (!s) return M3_EINVAL;
    if (s->batch < 0 || s->seqlen < 0 || s->nheads < 1 || s->headdim < 1 || s->dstate < 2 ||
        (s->dstate & 1) || s->rank < 1)
        return M3_EINVAL;
    if (s->io != M3_F32 && s->io != M3_BF16) return M3_EINVAL;
    if ((s->flags & ~kAllFlags) != 0) return M3_EINVAL;
    if ((s->flags & M3_FLAG_PARTIAL_ROPE) && (s->rope_pairs < 0 || s->rope_pairs > s->dstate / 2)) return M3_EINVAL;
    if ((s->flags & M3_FLAG_BCNORM) && !(s->norm_eps >= 0.f)) return M3_EINVAL;
    if (step && s->seqlen != 1) return M3_EINVAL;
    if (s->dstate > 128 || s->headdim > 128 || s->rank > 8) return M3_EUNSUPPORTED;
    if (s->nheads > 65535 || s->batch > 65535) return M3_EUNSUPPORTED;
    if (!step) {
        if (s->chunk != 16 && s->chunk != 32 && s->chunk != 64 && s->chunk != 128) return M3_EUNSUPPORTED;
        if ((int64_t)s->chunk * s->rank > 128) return M3_EUNSUPPORTED;
    }
    return M3_OK;
}

m3_status check_inputs(const m3_inputs *in, bool need_data, int nr) {
    if (!in) return M3_EINVAL;
    if (need_data) {
        if (!in->x || !in->Bm || !in->Cm || !in->dt || !in->lam || (nr > 0 && !in->theta) || !in->A || !in->D)
            return M3_EINVAL;
    } else if (!in->A || !in->D) {
        return M3_EINVAL;
    }
    const void *ptrs[] = {in->x, in->Bm, in->Cm, in->dt, in->lam, in->theta, in->A, in->D,
                          in->b_norm_w, in->c_norm_w, in->b_bias, in->c_bias, in->dt_bias, in->z};
    for (const void *p : ptrs)
        if (!aligned16(p)) return M3_EINVAL;
    return M3_OK;
}

// The angle array may be NULL when no pair rotates (it then holds nothing).
m3_status check_state(const m3_state *st, bool required, int nr) {
    if (!st) return required ? M3_EINVAL : M3_OK;
    if (!st->h || !st->prev_B || !st->prev_x || (nr > 0 && !st->angle)) return M3_EINVAL;
    if (!aligned16(st->h) || !aligned16(st->prev_B) || !aligned16(st->prev_x) || !aligned16(st->angle))
        return M3_EINVAL;
    return M3_OK;
}

// Effective row strides (elements between tokens b*T + t) of x, B, C, dt, lambda, theta, A,
// z and y: the caller's, or the contiguous row length for 0.  A stride shorter than its row
// gives M3_EINVAL, one of 2^24 or more M3_EUNSUPPORTED.
enum { kRsX, kRsB, kRsC, kRsDt, kRsLam, kRsTh, kRsA, kRsZ, kRsY, kRsCount };
struct RowStrides {
    int64_t v[kRsCount];
    bool contiguous_bc;  // B and C are contiguous [B, T, H, N, R]
    bool any;            // a caller stride differs from the contiguous one
};
m3_status row_strides(const m3_shape *s, const m3_inputs *in, RowStrides &rs) {
    const int64_t H = s->nheads, P = s->headdim, N = s->dstate, R = s->rank;
    const int64_t nr = rotated_pairs(s);
    const int64_t rx = in->mimo_x ? 1 : R, rz = in->mimo_z ? 1 : R, ry = in->mimo_o ? 1 : R;
    const int64_t row[kRsCount] = {H * P * rx, H * N * R, H * N * R, H, H, H * nr, H, H * P * rz, H * P * ry};
    const int64_t given[kRsCount] = {in->x_stride, in->B_stride, in->C_stride, in->dt_stride, in->lam_stride,
                                     in->theta_stride, in->A_stride, in->z_stride, 0};
    rs.any = false;
    for (int k = 0; k < kRsCount; ++k) {
        const int64_t g = given[k];
        if (g < 0 || (g != 0 && g < row[k])) return M3_EINVAL;
        if (g >= (int64_t)1 << 24) return M3_EUNSUPPORTED;
        rs.v[k] = g ? g : row[k];
        if (rs.v[k] != row[k]) rs.any = true;
    }
    rs.contiguous_bc = rs.v[kRsB] == row[kRsB] && rs.v[kRsC] == row[kRsC];
    return M3_OK;
}

// Checks of the MIMO projection vectors: only with a rank (MIMO or step call), mimo_z only
// with a gate input, 16-byte aligned.
m3_status check_mimo_proj(const m3_inputs *in, bool rank_call) {
    if (!in->mimo_x && !in->mimo_z && !in->mimo_o) return M3_OK;
    if (!rank_call) return M3_EINVAL;
    if (in->mimo_z && !in->z) return M3_EINVAL;
    if (!aligned16(in->mimo_x) || !aligned16(in->mimo_z) || !aligned16(in->mimo_o)) return M3_EINVAL;
    return M3_OK;
}

// Blocks, segments and workspace of one scan.
struct Plan {
    int TB, nblk, nseg, bps, ncg, nsub, sbps;
    size_t Sagg, lseg, pseg, cseg, Hin, total;
};

TileShape tile_of(const m3_shape *s) {
    TileShape ts;
    ts.np = pow2_at_least(s->dstate, 32);
    ts.pp = pow2_at_least(s->headdim < 64 ? s->headdim : 64, 32);
    const bool v8 = (s->dstate % 8) == 0 && (s->headdim % 8) == 0;
    ts.mode = m3::kTileGen;
    // the rank-1 path loads the angles of four pairs per 16-byte access
    if (v8 && s->rank == 1 && rotated_pairs(s) % 4 == 0) ts.mode = m3::kTileVec;
    else if (v8 && s->io == M3_BF16 && (s->rank == 2 || s->rank == 4 || s->rank == 8)) ts.mode = m3::kTileMimo;
    return ts;
}

// The kernel variant a call runs: the shape's, except that row strides whose byte size is not
// a multiple of 16, B and C rows of different strides, or the MIMO projections at rank 1, need
// the element-load path, and the interleaved-rank path needs 16-byte rows of its (possibly
// rank-free) x and z.  (The plan's segments follow the shape's variant, so the workspace size
// depends on the shape alone.)
TileShape kernel_tile(const m3_shape *s, const m3_inputs *in, const RowStrides &rs) {
    TileShape ts = tile_of(s);
    const int es = s->io == M3_BF16 ? 2 : 4;
    auto a16 = [&](int k) { return (rs.v[k] * es) % 16 == 0; };
    const bool rows16 = a16(kRsX) && a16(kRsB) && rs.v[kRsC] == rs.v[kRsB] && (!in->z || a16(kRsZ));
    const bool proj = in->mimo_x || in->mimo_z || in->mimo_o;
    if (ts.mode == m3::kTileVec && (proj || !rows16 || rs.v[kRsTh] % 4 != 0)) ts.mode = m3::kTileGen;
    if (ts.mode == m3::kTileMimo && !rows16) ts.mode = m3::kTileGen;
    ts.pj = proj;
    // reached with the flag only through the native half-split path (native_half_split)
    ts.hs = (s->flags & M3_FLAG_HALF_SPLIT) != 0 && ts.mode == m3::kTileVec;
    return ts;
}

Plan plan_of(const m3_shape *s) {
    Plan pl{};
    const int64_t T = s->seqlen;
    const TileShape ts0 = tile_of(s);
    pl.ncg = (s->headdim + ts0.pp - 1) / ts0.pp;
    const int64_t BH = s->batch * (int64_t)s->nheads * pl.ncg;  // independent (sequence, column group) pairs
    // tokens per 64-row block: the chunk, capped so chunk * rank fits the block
    const int cap = m3::kBlockRows / s->rank;
    pl.TB = s->chunk < cap ? s->chunk : cap;
    if (pl.TB < 1) pl.TB = 1;
    pl.nblk = (int)(T > 0 ? (T + pl.TB - 1) / pl.TB : 0);
    // segments: enough workgroups to fill the 256 compute units at the LDS occupancy
    const TileShape ts = tile_of(s);
    const size_t lds = m3::seg_kernel_lds_bytes(true, s->io == M3_BF16, ts);
    int per_cu = lds ? (int)((160 * 1024) / lds) : 1;
    if (per_cu < 1) per_cu = 1;
    if (per_cu > 4) per_cu = 4;
    const int64_t target = 256LL * per_cu;
    int64_t nseg = BH > 0 ? (target + BH - 1) / BH : 1;
    if (nseg > 16) nseg = 16;
    if (nseg > pl.nblk) nseg = pl.nblk;
    if (nseg < 1) nseg = 1;
    pl.bps = (int)((pl.nblk + nseg - 1) / nseg);
    if (pl.bps < 1) pl.bps = 1;
    pl.nseg = pl.nblk > 0 ? (pl.nblk + pl.bps - 1) / pl.bps : 1;
    // state sub-segments over the blocks of segments 0 .. nseg-2: halve them (while the
    // length stays a whole number of blocks) until about three state workgroups per unit,
    // six with ranks above 1 (measured faster there) (only with long segments: splitting
    // then pays for the extra prefix launch; otherwise one sub-segment per segment and the
    // output kernel folds the aggregates itself)
    pl.sbps = pl.bps;
    const int64_t sub_wgs = s->rank > 1 ? 1536 : 768;
    if (pl.bps >= 8 && pl.nseg > 1)
        while ((pl.sbps % 2) == 0 && BH * (pl.nseg - 1) * (pl.bps / pl.sbps) < sub_wgs &&
               (pl.nseg - 1) * (pl.bps / pl.sbps) < 32)
            pl.sbps /= 2;
    pl.nsub = (pl.nseg - 1) * (pl.bps / pl.sbps);
    const int64_t BHs = BH / pl.ncg;  // (batch, head) sequences
    const int64_t NSUB = BHs * (pl.nsub > 0 ? pl.nsub : 1);
    const int64_t np2 = ts.np / 2;
    size_t off = 0;
    pl.Sagg = off; off = align_up(off + sizeof(float) * (size_t)(BH * (pl.nsub > 0 ? pl.nsub : 1) * ts.np * ts.pp));
    pl.lseg = off; off = align_up(off + sizeof(float) * (size_t)NSUB);
    pl.pseg = off; off = align_up(off + sizeof(float) * (size_t)(NSUB * np2));
    pl.cseg = off; off = align_up(off + sizeof(float) * (size_t)(NSUB * np2 * 2));
    pl.Hin = off; off = align_up(off + sizeof(float) * (size_t)(BH * pl.nseg * ts.np * ts.pp));
    pl.total = (pl.nblk == 0 || BH == 0) ? 0 : off;
    return pl;
}

// Every argument check of a scan call but the workspace size (the half-split path runs these
// before its first permutation launch).
m3_status validate_scan(const m3_shape *s, const m3_inputs *in, const void *y, const m3_state *init,
                        const m3_state *fin, const void *ws, bool mimo) {
    m3_status rc = check_shape(s, false);
    if (rc != M3_OK) return rc;
    if (!mimo && s->rank != 1) return M3_EINVAL;
    rc = check_inputs(in, s->seqlen > 0 && s->batch > 0, rotated_pairs(s));
    if (rc != M3_OK) return rc;
    if ((rc = check_state(init, false, rotated_pairs(s))) != M3_OK) return rc;
    if ((rc = check_state(fin, false, rotated_pairs(s))) != M3_OK) return rc;
    if (s->seqlen > 0 && s->batch > 0 && !y) return M3_EINVAL;
    if (!aligned16(y)) return M3_EINVAL;
    if ((rc = check_mimo_proj(in, mimo)) != M3_OK) return rc;
    RowStrides rs;
    if ((rc = row_strides(s, in, rs)) != M3_OK) return rc;
    if ((s->flags & M3_FLAG_HALF_SPLIT) && !rs.contiguous_bc) return M3_EUNSUPPORTED;
    const TileShape ts = kernel_tile(s, in, rs);
    const bool bf = s->io == M3_BF16;
    if (m3::seg_kernel_lds_bytes(true, bf, ts) > 160 * 1024 || m3::seg_kernel_lds_bytes(false, bf, ts) > 160 * 1024)
        return M3_EUNSUPPORTED;
    if (!aligned16(ws)) return M3_EINVAL;
    return M3_OK;
}

m3_status scan_impl(const m3_shape *s, const m3_inputs *in, void *y, const m3_state *init,
                    m3_state *fin, void *ws, size_t ws_bytes, void *stream, bool mimo) {
    m3_status rc = validate_scan(s, in, y, init, fin, ws, mimo);
    if (rc != M3_OK) return rc;
    RowStrides rs;
    row_strides(s, in, rs);
    const TileShape ts = kernel_tile(s, in, rs);
    const bool bf = s->io == M3_BF16;
    const Plan pl = plan_of(s);
    if (pl.total > 0 && (!ws || ws_bytes < pl.total)) return M3_EWORKSPACE;

    ScanParams p;
    std::memset(&p, 0, sizeof p);
    p.dbg = debug_words();
    p.B = s->batch;
    p.T = s->seqlen;
    p.H = s->nheads;
    p.P = s->headdim;
    p.N = s->dstate;
    p.R = s->rank;
    p.TB = pl.TB;
    p.nblk = pl.nblk;
    p.nseg = pl.nseg;
    p.bps = pl.bps;
    p.nsub = pl.nsub;
    p.sbps = pl.sbps;
    p.ncg = pl.ncg;
    p.flags = s->flags;
    p.eps = s->norm_eps;
    p.nr = rotated_pairs(s);
    p.dtbias = in->dt_bias;
    p.z = in->z;
    p.x = in->x;
    p.Bm = in->Bm;
    p.Cm = in->Cm;
    p.dt = in->dt;
    p.lam = in->lam;
    p.theta = in->theta;
    p.A = in->A;
    p.D = in->D;
    p.bnw = in->b_norm_w;
    p.cnw = in->c_norm_w;
    p.bbias = in->b_bias;
    p.cbias = in->c_bias;
    p.mx = in->mimo_x;
    p.mz = in->mimo_z;
    p.mo = in->mimo_o;
    p.rsx = rs.v[kRsX];
    p.rsb = rs.v[kRsB];
    p.rsc = rs.v[kRsC];
    p.rsdt = rs.v[kRsDt];
    p.rslam = rs.v[kRsLam];
    p.rsth = rs.v[kRsTh];
    p.rsa = rs.v[kRsA];
    p.rsz = rs.v[kRsZ];
    p.rsy = rs.v[kRsY];
    p.y = y;
    if (init) {
        p.h0 = init->h;
        p.pB0 = init->prev_B;
        p.px0 = init->prev_x;
        p.ang0 = init->angle;
    }
    if (fin) {
        p.h1 = fin->h;
        p.pB1 = fin->prev_B;
        p.px1 = fin->prev_x;
        p.ang1 = fin->angle;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (p.B == 0) return M3_OK;
    if (p.T == 0) {
        if (!fin) return M3_OK;
        return m3::launch_fill_state(p, st) == hipSuccess ? M3_OK : M3_EHIP;
    }
    char *base = static_cast<char *>(ws);
    p.Sagg = reinterpret_cast<float *>(base + pl.Sagg);
    p.lseg = reinterpret_cast<float *>(base + pl.lseg);
    p.pseg = reinterpret_cast<float *>(base + pl.pseg);
    p.cseg = reinterpret_cast<float *>(base + pl.cseg);
    p.np2 = ts.np / 2;
    p.pp = ts.pp;
    // incoming states per segment from the prefix kernel when the state is split finer than
    // the segments; otherwise the output kernel assembles them itself
    const bool prefix = p.sbps < p.bps;
    if (ts.hs && prefix) return M3_EINVAL;  // (native_half_split excludes it)
    p.Hin = prefix ? reinterpret_cast<float *>(base + pl.Hin) : nullptr;
    if (p.nsub > 0 && m3::launch_seg_state(bf, ts, p, st) != hipSuccess) return M3_EHIP;
    if (prefix && m3::launch_seg_prefix(ts, p, st) != hipSuccess) return M3_EHIP;
    if (m3::launch_seg_output(bf, ts, p, st) != hipSuccess) return M3_EHIP;
    return M3_OK;
}

struct BwdPlan {
    int nck, pw;
    size_t Sst, Ust, lsum, phic, thst, G0w, hfin, tot, dsc, deta0, part;
    size_t total;
};

// Chunks of 64 (token, rank) rows; per chunk a state and an adjoint (N x P fp32 each).
BwdPlan bwd_plan_of(const m3_shape *s) {
    BwdPlan pl{};
    const int64_t BH = s->batch * (int64_t)s->nheads, T = s->seqlen;
    const int N = s->dstate, R = s->rank, N2 = N / 2, P = s->headdim;
    const int qt = 64 / R;
    pl.nck = T > 0 ? (int)((T + qt - 1) / qt) : 1;
    pl.pw = 3 + 2 * N + 2 * R * N;
    const int64_t C = BH * pl.nck;
    size_t off = 0;
    auto take = [&](size_t &at, int64_t floats) { at = off; off = align_up(off + sizeof(float) * (size_t)floats); };
    take(pl.Sst, C * N * P);
    take(pl.Ust, C * N * P);
    take(pl.lsum, C);
    take(pl.phic, C * N2);
    take(pl.thst, BH * N2);
    take(pl.G0w, BH * N * P);
    take(pl.hfin, BH * N * P);
    take(pl.tot, C * N2);
    take(pl.dsc, BH * T * 3);
    take(pl.deta0, BH);
    take(pl.part, C * pl.pw);
    pl.total = (T == 0 || BH == 0) ? 0 : off;
    return pl;
}

// Every argument check of a gradient call but the workspace size.
m3_status validate_bwd(const m3_shape *s, const m3_inputs *in, const void *dy, const m3_state *init,
                       const m3_state *dfin, const m3_grads *g, const m3_state *dinit, const void *ws) {
    m3_status rc = check_shape(s, false);
    if (rc != M3_OK) return rc;
    const int nr = rotated_pairs(s);
    const bool data = s->seqlen > 0 && s->batch > 0;
    if ((rc = check_inputs(in, data, nr)) != M3_OK) return rc;
    if ((rc = check_state(init, false, nr)) != M3_OK) return rc;
    if ((rc = check_state(dfin, false, nr)) != M3_OK) return rc;
    if ((rc = check_state(dinit, false, nr)) != M3_OK) return rc;
    if (!g) return M3_EINVAL;
    if (data && !dy) return M3_EINVAL;
    if (in->z && data && !g->dz) return M3_EINVAL;
    const void *ptrs[] = {dy, g->dx, g->dB, g->dC, g->ddt, g->dlam, g->dtheta, g->dA, g->dD, g->db_norm_w,
                          g->dc_norm_w, g->db_bias, g->dc_bias, g->ddt_bias, g->dz};
    for (const void *q : ptrs)
        if (!aligned16(q)) return M3_EINVAL;
    if (!aligned16(ws)) return M3_EINVAL;
    RowStrides rs;
    if ((rc = row_strides(s, in, rs)) != M3_OK) return rc;
    if (rs.any || in->mimo_x || in->mimo_z || in->mimo_o) return M3_EUNSUPPORTED;
    return M3_OK;
}

m3_status bwd_impl(const m3_shape *s, const m3_inputs *in, const void *dy, const m3_state *init,
                   const m3_state *dfin, m3_grads *g, m3_state *dinit, void *ws, size_t ws_bytes, void *stream) {
    m3_status rc = validate_bwd(s, in, dy, init, dfin, g, dinit, ws);
    if (rc != M3_OK) return rc;
    const int nr = rotated_pairs(s);
    const BwdPlan pl = bwd_plan_of(s);
    if (pl.total > 0 && (!ws || ws_bytes < pl.total)) return M3_EWORKSPACE;
    if (s->batch == 0) return M3_OK;
    m3::BwdParams p;
    std::memset(&p, 0, sizeof p);
    p.dbg = debug_words();
    p.B = s->batch;
    p.T = s->seqlen;
    p.H = s->nheads;
    p.P = s->headdim;
    p.N = s->dstate;
    p.R = s->rank;
    p.flags = s->flags;
    p.eps = s->norm_eps;
    p.nr = nr;
    p.hs = (s->flags & M3_FLAG_HALF_SPLIT) ? 1 : 0;  // (reached with the flag only through native_half_split_bwd)
    p.x = in->x;
    p.Bm = in->Bm;
    p.Cm = in->Cm;
    p.dt = in->dt;
    p.lam = in->lam;
    p.theta = in->theta;
    p.A = in->A;
    p.D = in->D;
    p.bnw = in->b_norm_w;
    p.cnw = in->c_norm_w;
    p.bbias = in->b_bias;
    p.cbias = in->c_bias;
    p.dtbias = in->dt_bias;
    p.z = in->z;
    if (init) {
        p.h0 = init->h;
        p.pB0 = init->prev_B;
        p.px0 = init->prev_x;
        p.ang0 = init->angle;
    }
    p.dy = dy;
    if (dfin) {
        p.dh1 = dfin->h;
        p.dpB1 = dfin->prev_B;
        p.dpx1 = dfin->prev_x;
        p.dang1 = dfin->angle;
    }
    p.dx = g->dx;
    p.dB = g->dB;
    p.dC = g->dC;
    p.dz = g->dz;
    p.ddt = g->ddt;
    p.dlam = g->dlam;
    p.dtheta = g->dtheta;
    const bool atok = (s->flags & M3_FLAG_A_PER_TOKEN) != 0;
    p.dAt = atok ? g->dA : nullptr;
    p.dA = atok ? nullptr : g->dA;
    p.dD = g->dD;
    p.dbnw = g->db_norm_w;
    p.dcnw = g->dc_norm_w;
    p.dbb = g->db_bias;
    p.dcb = g->dc_bias;
    p.ddtb = g->ddt_bias;
    if (dinit) {
        p.dh0 = dinit->h;
        p.dpB0 = dinit->prev_B;
        p.dpx0 = dinit->prev_x;
        p.dang0 = dinit->angle;
    }
    p.nck = pl.nck;
    {
        const int e = s->io == M3_BF16 ? 8 : 4;
        p.vec = (s->headdim * s->rank) % e == 0 && (s->dstate * s->rank) % e == 0 && nr % 4 == 0;
    }
    p.pw = pl.pw;
    char *base = static_cast<char *>(ws);
    auto at = [&](size_t off) { return pl.total ? reinterpret_cast<float *>(base + off) : nullptr; };
    p.Sst = at(pl.Sst);
    p.Ust = at(pl.Ust);
    p.lsum = at(pl.lsum);
    p.phic = at(pl.phic);
    p.thst = at(pl.thst);
    p.G0w = at(pl.G0w);
    p.hfin = at(pl.hfin);
    p.tot = at(pl.tot);
    p.dsc = at(pl.dsc);
    p.deta0 = at(pl.deta0);
    p.part = at(pl.part);
    return m3::launch_bwd(s->io == M3_BF16, p, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? M3_OK
                                                                                                     : M3_EHIP;
}

// ---------------------------------------------------------------- half-split pairing
// The kernels pair components (2i, 2i + 1).  A half-split call (pairs (i, i + N/2)) runs the
// same path on copies in the workspace with the N axis permuted: B, C, gains, biases and the
// N rows of the states in, the N-indexed outputs back.  The copies follow the plain call's
// workspace, one 256-byte aligned slot per tensor:
//   B, C, gains, biases (inputs); H0/PB0 the initial state's h / prev_B; H1/PB1 the final
//   state's (scan) or its gradients (gradient call); H2/PB2 the initial state's gradients;
//   DB .. DCB the gradients of B, C, the gains and the biases.
enum HsSlot {
    kHsB, kHsC, kHsBnw, kHsCnw, kHsBb, kHsCb, kHsH0, kHsPb0, kHsH1, kHsPb1,
    kHsH2, kHsPb2, kHsDB, kHsDC, kHsDBnw, kHsDCnw, kHsDBb, kHsDCb, kHsCount
};
struct HsLayout {
    size_t off[kHsCount];
    size_t total;
};
HsLayout hs_layout(const m3_shape *s, bool bwd) {
    HsLayout l{};
    const int64_t BTH = s->batch * s->seqlen * (int64_t)s->nheads, BH = s->batch * (int64_t)s->nheads;
    const int64_t N = s->dstate, R = s->rank, P = s->headdim, H = s->nheads;
    const size_t es = s->io == M3_BF16 ? 2 : 4;
    const size_t bc = BTH * N * R * es, g = N * 4, bi = H * R * N * 4, hs = BH * N * P * 4, pb = BH * N * R * 4;
    const size_t bytes[kHsCount] = {bc, bc, g, g, bi, bi, hs, pb, hs, pb,
                                    bwd ? hs : 0, bwd ? pb : 0, bwd ? bc : 0, bwd ? bc : 0,
                                    bwd ? g : 0, bwd ? g : 0, bwd ? bi : 0, bwd ? bi : 0};
    size_t off = 0;
    for (int k = 0; k < kHsCount; ++k) {
        l.off[k] = off;
        off = align_up(off + bytes[k]);
    }
    l.total = off;
    return l;
}

// A call with no tokens (or no batch) only copies the state, which does not depend on the
// pairing: no workspace, also with the half-split pairing.
bool no_tokens(const m3_shape *s) { return s->seqlen == 0 || s->batch == 0; }

size_t scan_ws_bytes(const m3_shape *s) {
    if (!(s->flags & M3_FLAG_HALF_SPLIT) || no_tokens(s)) return plan_of(s).total;
    m3_shape s2 = *s;
    s2.flags &= ~M3_FLAG_HALF_SPLIT;
    return align_up(plan_of(&s2).total) + hs_layout(s, false).total;
}

size_t bwd_ws_bytes(const m3_shape *s) {
    if (!(s->flags & M3_FLAG_HALF_SPLIT) || no_tokens(s)) return bwd_plan_of(s).total;
    m3_shape s2 = *s;
    s2.flags &= ~M3_FLAG_HALF_SPLIT;
    return align_up(bwd_plan_of(&s2).total) + hs_layout(s, true).total;
}

// Permutations of one call's N-indexed tensors between the caller's buffers and the slots.
struct HsPerm {
    const m3_shape *s;
    char *w;
    HsLayout hl;
    hipStream_t st;
    hipError_t e = hipSuccess;
    void *slot(int k) const { return w + hl.off[k]; }
    // [outer][N][inner] from src into slot k (to the kernels' order); returns the slot, or NULL
    template <class T>
    T *in(const T *src, int k, int64_t outer, int inner, int es) {
        if (!src) return nullptr;
        if (e == hipSuccess) e = m3::launch_perm_n(src, slot(k), outer, s->dstate, inner, es, true, st);
        return static_cast<T *>(slot(k));
    }
    // slot k back into dst (the caller's order)
    void out(int k, void *dst, int64_t outer, int inner, int es) {
        if (dst && e == hipSuccess) e = m3::launch_perm_n(slot(k), dst, outer, s->dstate, inner, es, false, st);
    }
};

// The rank-1 16-byte kernels pair (i, i + N/2) themselves when N fills their tile (64 or 128)
// and no prefix pass runs (the prefix kernel's fold keeps adjacent pairs); every other call
// with the half-split pairing runs on N-permuted copies.
bool native_half_split(const m3_shape *s, const m3_inputs *in) {
    const TileShape t = tile_of(s);
    if (t.mode != m3::kTileVec || s->dstate != t.np || t.np < 64) return false;
    const Plan pl = plan_of(s);
    if (pl.sbps < pl.bps) return false;
    RowStrides rs;
    if (row_strides(s, in, rs) != M3_OK) return false;
    const TileShape k = kernel_tile(s, in, rs);
    return k.mode == m3::kTileVec && !k.pj;
}

m3_status scan_half_split(const m3_shape *s, const m3_inputs *in, void *y, const m3_state *init, m3_state *fin,
                          void *ws, size_t ws_bytes, void *stream, bool mimo) {
    m3_status rc = validate_scan(s, in, y, init, fin, ws, mimo);
    if (rc != M3_OK) return rc;
    if (no_tokens(s)) {
        // only the state is copied (element by element): the pairing does not matter
        m3_shape s1 = *s;
        s1.flags &= ~M3_FLAG_HALF_SPLIT;
        return scan_impl(&s1, in, y, init, fin, ws, ws_bytes, stream, mimo);
    }
    // (the workspace is always the size m3_scan_workspace_bytes reports for the shape, which
    // holds the permuted copies whichever path runs)
    if (!ws || ws_bytes < scan_ws_bytes(s)) return M3_EWORKSPACE;
    if (native_half_split(s, in)) return scan_impl(s, in, y, init, fin, ws, ws_bytes, stream, mimo);
    m3_shape s2 = *s;
    s2.flags &= ~M3_FLAG_HALF_SPLIT;
    const size_t base = align_up(plan_of(&s2).total);
    HsPerm hp{s, nullptr, hs_layout(s, false), reinterpret_cast<hipStream_t>(stream)};
    if (!ws || ws_bytes < base + hp.hl.total) return M3_EWORKSPACE;
    hp.w = static_cast<char *>(ws) + base;
    const int64_t BTH = s->batch * s->seqlen * (int64_t)s->nheads, BH = s->batch * (int64_t)s->nheads;
    const int R = s->rank, P = s->headdim, H = s->nheads, es = s->io == M3_BF16 ? 2 : 4;
    m3_inputs in2 = *in;
    if (s->seqlen > 0) {
        in2.Bm = hp.in(static_cast<const char *>(in->Bm), kHsB, BTH, R, es);
        in2.Cm = hp.in(static_cast<const char *>(in->Cm), kHsC, BTH, R, es);
    }
    in2.b_norm_w = hp.in(in->b_norm_w, kHsBnw, 1, 1, 4);
    in2.c_norm_w = hp.in(in->c_norm_w, kHsCnw, 1, 1, 4);
    in2.b_bias = hp.in(in->b_bias, kHsBb, (int64_t)H * R, 1, 4);
    in2.c_bias = hp.in(in->c_bias, kHsCb, (int64_t)H * R, 1, 4);
    m3_state init2{}, fin2{};
    if (init) {
        init2 = *init;
        init2.h = hp.in(init->h, kHsH0, BH, P, 4);
        init2.prev_B = hp.in(init->prev_B, kHsPb0, BH, R, 4);
    }
    if (fin) {
        fin2 = *fin;
        fin2.h = static_cast<float *>(hp.slot(kHsH1));
        fin2.prev_B = static_cast<float *>(hp.slot(kHsPb1));
    }
    if (hp.e != hipSuccess) return M3_EHIP;
    rc = scan_impl(&s2, &in2, y, init ? &init2 : nullptr, fin ? &fin2 : nullptr, ws, base, stream, mimo);
    if (rc != M3_OK) return rc;
    if (fin) {
        hp.out(kHsH1, fin->h, BH, P, 4);
        hp.out(kHsPb1, fin->prev_B, BH, R, 4);
    }
    return hp.e == hipSuccess ? M3_OK : M3_EHIP;
}

// The gradient kernels pair (i, i + N/2) themselves when N is 64 or 128 (the two columns of a
// pair then sit in one lane of the chunk kernel's per-column passes); other sizes run on
// N-permuted copies.
bool native_half_split_bwd(const m3_shape *s) { return s->dstate == 64 || s->dstate == 128; }

m3_status bwd_half_split(const m3_shape *s, const m3_inputs *in, const void *dy, const m3_state *init,
                         const m3_state *dfin, m3_grads *g, m3_state *dinit, void *ws, size_t ws_bytes,
                         void *stream) {
    m3_status rc = validate_bwd(s, in, dy, init, dfin, g, dinit, ws);
    if (rc != M3_OK) return rc;
    if (no_tokens(s)) {
        // the gradients pass through element by element: the pairing does not matter
        m3_shape s1 = *s;
        s1.flags &= ~M3_FLAG_HALF_SPLIT;
        return bwd_impl(&s1, in, dy, init, dfin, g, dinit, ws, ws_bytes, stream);
    }
    // (the workspace is always the size m3_scan_bwd_workspace_bytes reports for the shape,
    // which holds the permuted copies whichever path runs)
    if (!ws || ws_bytes < bwd_ws_bytes(s)) return M3_EWORKSPACE;
    if (native_half_split_bwd(s)) return bwd_impl(s, in, dy, init, dfin, g, dinit, ws, ws_bytes, stream);
    m3_shape s2 = *s;
    s2.flags &= ~M3_FLAG_HALF_SPLIT;
    const size_t base = align_up(bwd_plan_of(&s2).total);
    HsPerm hp{s, nullptr, hs_layout(s, true), reinterpret_cast<hipStream_t>(stream)};
    if (!ws || ws_bytes < base + hp.hl.total) return M3_EWORKSPACE;
    hp.w = static_cast<char *>(ws) + base;
    const int64_t BTH = s->batch * s->seqlen * (int64_t)s->nheads, BH = s->batch * (int64_t)s->nheads;
    const int R = s->rank, P = s->headdim, H = s->nheads, es = s->io == M3_BF16 ? 2 : 4;
    m3_inputs in2 = *in;
    if (s->seqlen > 0) {
        in2.Bm = hp.in(static_cast<const char *>(in->Bm), kHsB, BTH, R, es);
        in2.Cm = hp.in(static_cast<const char *>(in->Cm), kHsC, BTH, R, es);
    }
    in2.b_norm_w = hp.in(in->b_norm_w, kHsBnw, 1, 1, 4);
    in2.c_norm_w = hp.in(in->c_norm_w, kHsCnw, 1, 1, 4);
    in2.b_bias = hp.in(in->b_bias, kHsBb, (int64_t)H * R, 1, 4);
    in2.c_bias = hp.in(in->c_bias, kHsCb, (int64_t)H * R, 1, 4);
    m3_state init2{}, dfin2{}, dinit2{};
    if (init) {
        init2 = *init;
        init2.h = hp.in(init->h, kHsH0, BH, P, 4);
        init2.prev_B = hp.in(init->prev_B, kHsPb0, BH, R, 4);
    }
    if (dfin) {
        dfin2 = *dfin;
        dfin2.h = hp.in(dfin->h, kHsH1, BH, P, 4);
        dfin2.prev_B = hp.in(dfin->prev_B, kHsPb1, BH, R, 4);
    }
    if (dinit) {
        dinit2 = *dinit;
        dinit2.h = static_cast<float *>(hp.slot(kHsH2));
        dinit2.prev_B = static_cast<float *>(hp.slot(kHsPb2));
    }
    m3_grads g2 = *g;
    if (g->dB) g2.dB = hp.slot(kHsDB);
    if (g->dC) g2.dC = hp.slot(kHsDC);
    if (g->db_norm_w) g2.db_norm_w = static_cast<float *>(hp.slot(kHsDBnw));
    if (g->dc_norm_w) g2.dc_norm_w = static_cast<float *>(hp.slot(kHsDCnw));
    if (g->db_bias) g2.db_bias = static_cast<float *>(hp.slot(kHsDBb));
    if (g->dc_bias) g2.dc_bias = static_cast<float *>(hp.slot(kHsDCb));
    if (hp.e != hipSuccess) return M3_EHIP;
    rc = bwd_impl(&s2, &in2, dy, init ? &init2 : nullptr, dfin ? &dfin2 : nullptr, &g2, dinit ? &dinit2 : nullptr,
                  ws, base, stream);
    if (rc != M3_OK) return rc;
    if (s->seqlen > 0) {
        hp.out(kHsDB, g->dB, BTH, R, es);
        hp.out(kHsDC, g->dC, BTH, R, es);
    }
    hp.out(kHsDBnw, g->db_norm_w, 1, 1, 4);
    hp.out(kHsDCnw, g->dc_norm_w, 1, 1, 4);
    hp.out(kHsDBb, g->db_bias, (int64_t)H * R, 1, 4);
    hp.out(kHsDCb, g->dc_bias, (int64_t)H * R, 1, 4);
    if (dinit) {
        hp.out(kHsH2, dinit->h, BH, P, 4);
        hp.out(kHsPb2, dinit->prev_B, BH, R, 4);
    }
    return hp.e == hipSuccess ? M3_OK : M3_EHIP;
}

// ---------------------------------------------------------------- library-owned scratch
// The workspace of m3_scan_noalloc: a file-scope device array, one copy per GPU, held by the
// loaded code object until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[M3_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch (looked up on the device's first call), or NULL.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

m3_status m3_scan_noalloc(const m3_shape *shape, const m3_inputs *in, void *y, const m3_state *init,
                          m3_state *final, void *stream) {
    // every argument check first, with the scratch standing in for the workspace
    m3_status rc = validate_scan(shape, in, y, init, final, nullptr, true);
    if (rc != M3_OK) return rc;
    if (scan_ws_bytes(shape) > (size_t)M3_STATIC_SCRATCH_BYTES) return M3_EWORKSPACE;
    void *ws = device_scratch();
    if (!ws) return M3_EHIP;
    if (shape->flags & M3_FLAG_HALF_SPLIT)
        return scan_half_split(shape, in, y, init, final, ws, M3_STATIC_SCRATCH_BYTES, stream, true);
    return scan_impl(shape, in, y, init, final, ws, M3_STATIC_SCRATCH_BYTES, stream, true);
}

size_t m3_scan_bwd_workspace_bytes(const m3_shape *shape) {
    if (!shape || shape->seqlen < 0 || shape->batch < 0 || shape->nheads < 1 || shape->headdim < 1 ||
        shape->dstate < 2 || shape->rank < 1 || shape->rank > 8 || (shape->dstate & 1) || shape->dstate > 128 ||
        shape->headdim > 128)
        return 0;
    return bwd_ws_bytes(shape);
}

m3_status m3_scan_bwd(const m3_shape *shape, const m3_inputs *in, const void *dy, const m3_state *init,
                      const m3_state *dfinal, m3_grads *grads, m3_state *dinit, void *ws, size_t ws_bytes,
                      void *stream) {
    if (shape && (shape->flags & M3_FLAG_HALF_SPLIT))
        return bwd_half_split(shape, in, dy, init, dfinal, grads, dinit, ws, ws_bytes, stream);
    return bwd_impl(shape, in, dy, init, dfinal, grads, dinit, ws, ws_bytes, stream);
}


size_t m3_scan_workspace_bytes(const m3_shape *shape) {
    if (!shape || shape->chunk < 1 || shape->seqlen < 0 || shape->batch < 0 || shape->nheads < 1 ||
        shape->headdim < 1 || shape->dstate < 2)
        return 0;
    if (shape->rank < 1 || shape->rank > 8 || (shape->dstate & 1) || shape->dstate > 128 || shape->headdim > 128)
        return 0;
    return scan_ws_bytes(shape);
}

m3_status m3_scan_siso(const m3_shape *shape, const m3_inputs *in, void *y, const m3_state *init,
                       m3_state *final, void *ws, size_t ws_bytes, void *stream) {
    if (shape && (shape->flags & M3_FLAG_HALF_SPLIT)) {
        if (shape->rank != 1) return M3_EINVAL;
        return scan_half_split(shape, in, y, init, final, ws, ws_bytes, stream, false);
    }
    return scan_impl(shape, in, y, init, final, ws, ws_bytes, stream, false);
}

m3_status m3_scan_mimo(const m3_shape *shape, const m3_inputs *in, void *y, const m3_state *init,
                       m3_state *final, void *ws, size_t ws_bytes, void *stream) {
    if (shape && (shape->flags & M3_FLAG_HALF_SPLIT))
        return scan_half_split(shape, in, y, init, final, ws, ws_bytes, stream, true);
    return scan_impl(shape, in, y, init, final, ws, ws_bytes, stream, true);
}

m3_status m3_step(const m3_shape *s, const m3_inputs *in, void *y, m3_state *state, void *stream) {
    m3_status rc = check_shape(s, true);
    if (rc != M3_OK) return rc;
    if ((rc = check_inputs(in, s->batch > 0, rotated_pairs(s))) != M3_OK) return rc;
    if ((rc = check_state(state, true, rotated_pairs(s))) != M3_OK) return rc;
    if (s->batch > 0 && !y) return M3_EINVAL;
    if (!aligned16(y)) return M3_EINVAL;
    if ((rc = check_mimo_proj(in, true)) != M3_OK) return rc;
    RowStrides rs;
    if ((rc = row_strides(s, in, rs)) != M3_OK) return rc;
    if (s->batch == 0) return M3_OK;
    StepParams p;
    std::memset(&p, 0, sizeof p);
    p.dbg = debug_words();
    p.B = s->batch;
    p.H = s->nheads;
    p.P = s->headdim;
    p.N = s->dstate;
    p.R = s->rank;
    p.flags = s->flags;
    p.eps = s->norm_eps;
    p.nr = rotated_pairs(s);
    p.dtbias = in->dt_bias;
    p.z = in->z;
    p.x = in->x;
    p.Bm = in->Bm;
    p.Cm = in->Cm;
    p.dt = in->dt;
    p.lam = in->lam;
    p.theta = in->theta;
    p.A = in->A;
    p.D = in->D;
    p.bnw = in->b_norm_w;
    p.cnw = in->c_norm_w;
    p.bbias = in->b_bias;
    p.cbias = in->c_bias;
    p.mx = in->mimo_x;
    p.mz = in->mimo_z;
    p.mo = in->mimo_o;
    p.rsx = rs.v[kRsX];
    p.rsb = rs.v[kRsB];
    p.rsc = rs.v[kRsC];
    p.rsdt = rs.v[kRsDt];
    p.rslam = rs.v[kRsLam];
    p.rsth = rs.v[kRsTh];
    p.rsa = rs.v[kRsA];
    p.rsz = rs.v[kRsZ];
    p.rsy = rs.v[kRsY];
    p.y = y;
    p.h = state->h;
    p.pB = state->prev_B;
    p.px = state->prev_x;
    p.ang = state->angle;
    return m3::launch_step(s->io == M3_BF16, p, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? M3_OK
               : M3_EHIP;
}

m3_status m3_debug_checks(uint32_t *failed, uint32_t *line) {
#ifdef M3_DEBUG
    unsigned int *d = debug_words();
    if (!d) return M3_EHIP;
    unsigned int h[2] = {0u, 0u};
    const unsigned int zero[2] = {0u, 0u};
    if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(h, d, sizeof h, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(d, zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
        return M3_EHIP;
    if (failed) *failed = h[0];
    if (line) *line = h[1];
    return M3_OK;
#else
    (void)failed;
    (void)line;
    return M3_EUNSUPPORTED;
#endif
}

const char *m3_status_str(m3_status status) {
    // a C caller may pass any int; read it as one (an out-of-range enum value is undefined in C++)
    int code;
    std::memcpy(&code, &status, sizeof code);
    switch (code) {
        case M3_OK: return "M3_OK: success";
        case M3_EINVAL: return "M3_EINVAL: invalid argument (NULL pointer, bad size, odd N, rank < 1, unknown flag, rope_pairs outside 0..N/2 or misaligned pointer)";
        case M3_EUNSUPPORTED: return "M3_EUNSUPPORTED: size or option outside the supported range (N, P <= 128, R <= 8, chunk in {16,32,64,128}, chunk*R <= 128, row strides below 2^24; the gradient call needs contiguous inputs without MIMO projections)";
        case M3_EWORKSPACE: return "M3_EWORKSPACE: workspace missing or smaller than m3_scan_workspace_bytes()";
        case M3_EHIP: return "M3_EHIP: a HIP launch failed";
    }
    return "unknown m3_status";
}

const char *m3_version(void) { return "0.2.0"; }

}  // extern "C"
