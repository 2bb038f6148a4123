// stub_launchers.cpp -- host-only stand-ins for the kernel launchers of libmamba3, for the
// sanitizer build of the host dispatch layer (m3_api.cpp).  TEST INFRASTRUCTURE ONLY.
//
// Each stub launches nothing: it checks the parameter block the dispatch layer built (sizes,
// plan invariants, and that every workspace array lies inside the workspace the driver
// registered) and counts the launch.  AddressSanitizer and UndefinedBehaviorSanitizer watch
// the dispatch code itself.
#include <cstdio>
#include <cstdint>

#include "m3_internal.hpp"

namespace {
const char *g_lo = nullptr, *g_hi = nullptr;
int g_failures = 0, g_launches = 0;

void fail(const char *what) {
    ++g_failures;
    std::fprintf(stderr, "stub check failed: %s\n", what);
}
// [p, p + bytes) inside the registered workspace
void in_ws(const void *p, int64_t bytes, const char *what) {
    if (bytes <= 0) return;
    const char *c = static_cast<const char *>(p);
    if (!c || c < g_lo || c + bytes > g_hi) fail(what);
    if (reinterpret_cast<uintptr_t>(c) % 16) fail(what);
}
}  // namespace

extern "C" void m3s_set_workspace(const void *lo, size_t bytes) {
    g_lo = static_cast<const char *>(lo);
    g_hi = g_lo + bytes;
}
extern "C" int m3s_failures() { return g_failures; }
extern "C" int m3s_launches() { return g_launches; }

namespace m3 {

// LDS of a segment kernel: a fixed stand-in (the real sizes depend on the compiled tiles)
size_t seg_kernel_lds_bytes(bool output, bool, const TileShape &ts) {
    return (output ? 48 * 1024 : 32 * 1024) + (ts.pj ? 8 * 1024 : 0);
}

static void check_scan(const ScanParams &p, const TileShape &ts, bool output) {
    ++g_launches;
    if (p.B <= 0 || p.T <= 0 || p.H <= 0 || p.P <= 0 || p.N <= 0 || p.R <= 0) fail("scan sizes");
    if (p.TB < 1 || p.TB * p.R > kBlockRows) fail("tokens per block");
    if ((int64_t)p.nblk * p.TB < p.T || (int64_t)(p.nblk - 1) * p.TB >= p.T) fail("block count");
    if (p.nseg < 1 || p.bps < 1 || (int64_t)p.nseg * p.bps < p.nblk || (int64_t)(p.nseg - 1) * p.bps >= p.nblk)
        fail("segments");
    if (p.sbps < 1 || p.bps % p.sbps) fail("sub-segments");
    if (ts.np < p.N || ts.pp < 1 || p.ncg * ts.pp < p.P) fail("tile");
    if (p.rsx <= 0 || p.rsb <= 0 || p.rsc <= 0 || p.rsdt <= 0 || p.rslam <= 0 || p.rsy <= 0) fail("strides");
    if (!p.x || !p.Bm || !p.Cm || !p.dt || !p.lam || !p.A || !p.D || !p.y) fail("inputs");
    const int64_t bh = p.B * p.H, np2 = p.np2;
    const int64_t tile = (int64_t)ts.np * ts.pp;
    if (p.nsub > 0) {
        in_ws(p.Sagg, bh * p.ncg * p.nsub * tile * 4, "Sagg");
        in_ws(p.lseg, bh * p.nsub * 4, "lseg");
        in_ws(p.pseg, bh * p.nsub * np2 * 4, "pseg");
        in_ws(p.cseg, bh * p.nsub * np2 * 8, "cseg");
    }
    if (p.Hin) in_ws(p.Hin, bh * p.ncg * p.nseg * tile * 4, "Hin");
    (void)output;
}

hipError_t launch_seg_state(bool, const TileShape &ts, const ScanParams &p, hipStream_t) {
    check_scan(p, ts, false);
    if (p.nsub < 1) fail("state launch without sub-segments");
    return hipSuccess;
}
hipError_t launch_seg_prefix(const TileShape &ts, const ScanParams &p, hipStream_t) {
    check_scan(p, ts, false);
    if (!p.Hin) fail("prefix launch without Hin");
    return hipSuccess;
}
hipError_t launch_seg_output(bool, const TileShape &ts, const ScanParams &p, hipStream_t) {
    check_scan(p, ts, true);
    return hipSuccess;
}
hipError_t launch_fill_state(const ScanParams &p, hipStream_t) {
    ++g_launches;
    if (!p.h1 || !p.pB1 || !p.px1) fail("fill_state outputs");
    return hipSuccess;
}
hipError_t launch_step(bool, const StepParams &p, hipStream_t) {
    ++g_launches;
    if (p.B <= 0 || p.H <= 0 || !p.x || !p.Bm || !p.Cm || !p.y || !p.h || !p.pB || !p.px) fail("step");
    if (p.rsx <= 0 || p.rsb <= 0 || p.rsc <= 0 || p.rsdt <= 0 || p.rslam <= 0 || p.rsy <= 0) fail("step strides");
    return hipSuccess;
}
hipError_t launch_bwd(bool, const BwdParams &p, hipStream_t) {
    ++g_launches;
    const int64_t bh = p.B * p.H, C = bh * p.nck, N = p.N, P = p.P, N2 = p.N / 2;
    if (bh <= 0) fail("bwd sizes");
    if (p.T == 0) {  // no tokens: the state gradients pass through, no workspace
        if (p.Sst || p.part) fail("bwd workspace without tokens");
        return hipSuccess;
    }
    if ((int64_t)p.nck * (64 / p.R) < p.T) fail("bwd plan");
    // the half-split pairing reaches the kernels exactly at N = 64 or 128 (other sizes run on
    // N-permuted copies with the flag cleared)
    const bool hsflag = (p.flags & kFlagHalfSplit) != 0;
    if (hsflag != (p.hs != 0) || (p.hs && p.N != 64 && p.N != 128)) fail("bwd half-split pairing");
    in_ws(p.Sst, C * N * P * 4, "Sst");
    in_ws(p.Ust, C * N * P * 4, "Ust");
    in_ws(p.lsum, C * 4, "lsum");
    in_ws(p.phic, C * N2 * 4, "phic");
    in_ws(p.thst, bh * N2 * 4, "thst");
    in_ws(p.G0w, bh * N * P * 4, "G0w");
    in_ws(p.hfin, bh * N * P * 4, "hfin");
    in_ws(p.tot, C * N2 * 4, "tot");
    in_ws(p.dsc, bh * p.T * 3 * 4, "dsc");
    in_ws(p.deta0, bh * 4, "deta0");
    in_ws(p.part, C * p.pw * 4, "part");
    return hipSuccess;
}
hipError_t launch_perm_n(const void *in, void *out, int64_t outer, int N, int inner, int esize, bool to_kernel,
                         hipStream_t) {
    ++g_launches;
    if (!in || !out || outer <= 0 || N <= 0 || inner <= 0 || (esize != 2 && esize != 4)) fail("perm_n");
    // the kernel-side copy always lives in the workspace
    in_ws(to_kernel ? out : in, outer * N * (int64_t)inner * esize, "perm_n workspace copy");
    return hipSuccess;
}

}  // namespace m3
