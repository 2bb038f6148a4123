// host_driver.cpp -- drives every entry point of libmamba3's host dispatch layer, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against the stub launchers
// (stub_launchers.cpp), over a seeded sweep of shapes, options, strides and MIMO projections,
// and over argument errors.  Exits non-zero when a stub check fails or an entry point returns
// an unexpected status.  TEST INFRASTRUCTURE ONLY.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "libmamba3.h"

extern "C" void m3s_set_workspace(const void *lo, size_t bytes);
extern "C" int m3s_failures();
extern "C" int m3s_launches();

namespace {

// Fake device arrays: 16-byte aligned host addresses that the stubs never dereference.
alignas(256) unsigned char g_dummy[4096];
void *D(int k) { return g_dummy + 256 * (k % 16); }
float *F(int k) { return reinterpret_cast<float *>(g_dummy + 256 * (k % 16)); }

int g_bad = 0;
void expect(bool ok, const char *what, int64_t a = 0, int64_t b = 0) {
    if (!ok) {
        ++g_bad;
        std::fprintf(stderr, "unexpected: %s (%lld, %lld)\n", what, (long long)a, (long long)b);
    }
}

// A workspace of exactly `bytes` (heap, so that ASan sees its bounds), registered with the stubs.
struct Ws {
    std::vector<unsigned char> buf;
    void *p = nullptr;
    explicit Ws(size_t bytes) : buf(bytes + 256) {
        uintptr_t a = (reinterpret_cast<uintptr_t>(buf.data()) + 255) & ~uintptr_t(255);
        p = reinterpret_cast<void *>(a);
        m3s_set_workspace(p, bytes);
    }
};

m3_inputs inputs(bool z, int proj, std::mt19937 &rng, const m3_shape &s, bool strided) {
    m3_inputs in;
    std::memset(&in, 0, sizeof in);
    in.x = D(0);
    in.Bm = D(1);
    in.Cm = D(2);
    in.dt = F(3);
    in.lam = F(4);
    in.theta = F(5);
    in.A = F(6);
    in.D = F(7);
    if (rng() % 2) { in.b_norm_w = F(8); in.c_norm_w = F(9); }
    if (rng() % 2) { in.b_bias = F(10); in.c_bias = F(11); }
    if (s.flags & M3_FLAG_DT_SOFTPLUS) in.dt_bias = F(12);
    if (z) in.z = D(13);
    if (proj & 1) in.mimo_x = F(14);
    if ((proj & 2) && z) in.mimo_z = F(15);
    if (proj & 4) in.mimo_o = F(1);
    if (strided) {
        const int64_t H = s.nheads, P = s.headdim, N = s.dstate, R = s.rank;
        const int64_t extra = 8 * (1 + rng() % 3) + (rng() % 2);
        in.x_stride = H * P * (in.mimo_x ? 1 : R) + extra;
        in.B_stride = H * N * R + extra;
        in.C_stride = in.B_stride + 8 * (rng() % 2);
        in.dt_stride = H + rng() % 5;
        in.lam_stride = H + rng() % 5;
        in.theta_stride = H * (N / 2) + 4 * (rng() % 2);
        in.A_stride = H + 1;
        in.z_stride = z ? H * P * (in.mimo_z ? 1 : R) + extra : 0;
    }
    return in;
}

m3_state state(int base) {
    m3_state st;
    st.h = F(base);
    st.prev_B = F(base + 1);
    st.prev_x = F(base + 2);
    st.angle = F(base + 3);
    return st;
}

}  // namespace

int main() {
    std::mt19937 rng(12345);
    const int chunks[] = {16, 32, 64, 128};
    int ok_calls = 0, unsupported = 0;
    for (int it = 0; it < 3000; ++it) {
        m3_shape s;
        std::memset(&s, 0, sizeof s);
        s.batch = (int64_t)(rng() % 4);
        const int tmode = rng() % 6;
        s.seqlen = tmode == 0 ? 0 : tmode == 1 ? 1 : tmode < 4 ? (int64_t)(rng() % 300) : (int64_t)(rng() % 5000);
        s.nheads = 1 + rng() % 5;
        const int pc[] = {1, 5, 8, 16, 24, 32, 40, 64, 96, 128};
        s.headdim = pc[rng() % 10];
        const int nc[] = {2, 6, 8, 16, 24, 32, 64, 96, 128};
        s.dstate = nc[rng() % 9];
        s.rank = (rng() % 3 == 0) ? 1 + rng() % 8 : 1;
        s.chunk = chunks[rng() % 4];
        if (s.chunk * s.rank > 128) s.chunk = 16;
        s.io = rng() % 2 ? M3_BF16 : M3_F32;
        s.flags = M3_FLAG_BCNORM;
        if (rng() % 3 == 0) { s.flags |= M3_FLAG_PARTIAL_ROPE; s.rope_pairs = rng() % (s.dstate / 2 + 1); }
        if (rng() % 3 == 0) s.flags |= M3_FLAG_A_PER_TOKEN;
        if (rng() % 3 == 0) s.flags |= M3_FLAG_DT_SOFTPLUS;
        if (rng() % 3 == 0) s.flags |= M3_FLAG_LAM_SIGMOID;
        if (rng() % 4 == 0) s.flags |= M3_FLAG_HALF_SPLIT;
        s.norm_eps = 1e-5f;
        const bool z = rng() % 2;
        const int proj = (rng() % 3 == 0) ? (int)(rng() % 8) : 0;
        const bool strided = rng() % 3 == 0 && !(s.flags & M3_FLAG_HALF_SPLIT);
        m3_inputs in = inputs(z, proj, rng, s, strided);
        m3_state init = state(0), fin = state(4);
        const bool mimo = s.rank > 1 || proj || rng() % 2;

        // forward scan with a workspace of exactly the reported size
        const size_t wsb = m3_scan_workspace_bytes(&s);
        expect(s.seqlen > 0 && s.batch > 0 ? wsb > 0 : wsb == 0, "workspace size", s.seqlen, (int64_t)wsb);
        {
            Ws ws(wsb);
            const m3_status rc = mimo ? m3_scan_mimo(&s, &in, D(3), rng() % 2 ? &init : nullptr,
                                                     rng() % 2 ? &fin : nullptr, wsb ? ws.p : nullptr, wsb, nullptr)
                                      : m3_scan_siso(&s, &in, D(3), &init, &fin, wsb ? ws.p : nullptr, wsb, nullptr);
            expect(rc == M3_OK || rc == M3_EUNSUPPORTED, "scan status", rc, it);
            ok_calls += rc == M3_OK;
            unsupported += rc == M3_EUNSUPPORTED;
            if (wsb > 0) {
                // one byte short is always refused
                expect((mimo ? m3_scan_mimo(&s, &in, D(3), nullptr, nullptr, ws.p, wsb - 1, nullptr)
                             : m3_scan_siso(&s, &in, D(3), nullptr, nullptr, ws.p, wsb - 1, nullptr)) != M3_OK,
                       "short workspace accepted", it);
            }
        }
        // gradient call (contiguous inputs, no projections)
        if (!strided && !proj) {
            const size_t bwb = m3_scan_bwd_workspace_bytes(&s);
            Ws ws(bwb);
            m3_grads g;
            std::memset(&g, 0, sizeof g);
            g.dx = D(1);
            g.dB = D(2);
            g.dC = D(3);
            g.ddt = F(4);
            g.dlam = F(5);
            g.dtheta = F(6);
            g.dA = F(7);
            g.dD = F(8);
            g.dz = z ? D(9) : nullptr;
            m3_state dfin = state(8), dinit = state(12);
            const m3_status rc = m3_scan_bwd(&s, &in, D(10), &init, rng() % 2 ? &dfin : nullptr, &g, &dinit,
                                             bwb ? ws.p : nullptr, bwb, nullptr);
            expect(rc == M3_OK || rc == M3_EUNSUPPORTED, "bwd status", rc, it);
        }
        // decode step
        {
            m3_shape s1 = s;
            s1.seqlen = 1;
            if (s1.batch == 0) s1.batch = 1;
            m3_inputs in1 = inputs(z, proj, rng, s1, strided);
            m3_state st = state(0);
            const m3_status rc = m3_step(&s1, &in1, D(3), &st, nullptr);
            expect(rc == M3_OK || rc == M3_EUNSUPPORTED, "step status", rc, it);
        }
    }
    // argument errors (a sample; the Python host tests cover them one by one)
    {
        m3_shape s;
        std::memset(&s, 0, sizeof s);
        s.batch = 2; s.seqlen = 100; s.nheads = 2; s.headdim = 64; s.dstate = 64; s.rank = 1; s.chunk = 64;
        s.io = M3_BF16; s.flags = M3_FLAG_BCNORM; s.norm_eps = 1e-5f;
        std::mt19937 r2(7);
        m3_inputs in = inputs(false, 0, r2, s, false);
        Ws ws(m3_scan_workspace_bytes(&s));
        expect(m3_scan_siso(&s, nullptr, D(3), nullptr, nullptr, ws.p, 1 << 30, nullptr) == M3_EINVAL, "null inputs");
        expect(m3_scan_siso(nullptr, &in, D(3), nullptr, nullptr, ws.p, 1 << 30, nullptr) == M3_EINVAL, "null shape");
        in.x_stride = 3;
        expect(m3_scan_siso(&s, &in, D(3), nullptr, nullptr, ws.p, 1 << 30, nullptr) == M3_EINVAL, "short stride");
        in.x_stride = 0;
        in.mimo_o = F(1);
        expect(m3_scan_siso(&s, &in, D(3), nullptr, nullptr, ws.p, 1 << 30, nullptr) == M3_EINVAL, "siso projection");
        expect(std::strlen(m3_status_str((m3_status)99)) > 0 && std::strlen(m3_version()) > 0, "strings");
    }
    std::printf("calls ok %d, unsupported %d, launches %d, stub failures %d, unexpected %d\n", ok_calls, unsupported,
                m3s_launches(), m3s_failures(), g_bad);
    return (m3s_failures() || g_bad || ok_calls < 1000) ? 1 : 0;
}
