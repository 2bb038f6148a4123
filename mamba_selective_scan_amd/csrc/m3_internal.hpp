// m3_internal.hpp -- parameter block and launcher declarations shared by the
// host dispatch (m3_api.cpp) and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

struct ScanParams {
    // sizes
    int64_t B, T;
    int H, P, N, R, Q;  // Q = tokens per chunk
    int nchunks;
    uint32_t flags;
    float eps;
    // inputs
    const void *x, *Bm, *Cm;
    const float *dt, *lam, *theta, *A, *D;
    const float *bnw, *cnw, *bbias, *cbias;
    void *y;
    // carried state
    const float *h0, *pB0, *px0, *ang0;  // initial (NULL = zeros)
    float *h1, *pB1, *px1, *ang1;        // final (NULL = not requested)
    // workspace
    float *S;      // [B][H][C][P][N]  chunk states (in place: states entering each chunk)
    float *decay;  // [B][H][C]        exp(sum of log alpha over the chunk)
    float *phi;    // [B][H][C][N/2]   chunk angle totals
    float *cphi;   // [B][H][C][N/2]   cos of phi
    float *sphi;   // [B][H][C][N/2]   sin of phi
    float *thfin;  // [B][H][N/2]      final cumulative angle, in [0, 2 pi)
};

struct StepParams {
    int64_t B;
    int H, P, N, R;
    uint32_t flags;
    float eps;
    const void *x, *Bm, *Cm;
    const float *dt, *lam, *theta, *A, *D;
    const float *bnw, *cnw, *bbias, *cbias;
    void *y;
    float *h, *pB, *px, *ang;
};

enum { MODE_STATE = 0, MODE_OUTPUT = 1 };

// Tile shape chosen by the host: rows per chunk (Q*R padded), padded N, padded P.
struct TileShape {
    int rows, np, pp;
};

// Launchers (return hipSuccess or the launch error).  Defined in the kernel TUs.
hipError_t launch_chunk_kernel(int mode, bool bf16, const TileShape &ts, const ScanParams &p,
                               hipStream_t stream);
size_t chunk_kernel_lds_bytes(int mode, bool bf16, const TileShape &ts);
hipError_t launch_state_pass(const ScanParams &p, hipStream_t stream);
hipError_t launch_fill_state(const ScanParams &p, hipStream_t stream);
hipError_t launch_step(bool bf16, const StepParams &p, hipStream_t stream);

}  // namespace m3
