// m3_scan.hip -- choice of the scan kernel variant (io type x load path) and the
// segment prefix kernel.
#define M3_WITH_PREFIX_KERNEL
#include "m3_scan_impl.hpp"

namespace m3 {

#define M3_DECLARE(NAME)                                                                              \
    hipError_t NAME##_launch(bool output, const TileShape &ts, const ScanParams &p, hipStream_t st); \
    size_t NAME##_bytes(bool output, const TileShape &ts);
M3_DECLARE(scan_bf16_vec)
M3_DECLARE(scan_bf16_gen)
M3_DECLARE(scan_f32_vec)
M3_DECLARE(scan_f32_gen)
M3_DECLARE(scan_bf16_mimo)
#undef M3_DECLARE

size_t seg_kernel_lds_bytes(bool output, bool bf16, const TileShape &ts) {
    if (bf16) {
        if (ts.mode == kTileVec) return scan_bf16_vec_bytes(output, ts);
        if (ts.mode == kTileMimo) return scan_bf16_mimo_bytes(output, ts);
        return scan_bf16_gen_bytes(output, ts);
    }
    return ts.mode == kTileVec ? scan_f32_vec_bytes(output, ts) : scan_f32_gen_bytes(output, ts);
}

static hipError_t launch(bool output, bool bf16, const TileShape &ts, const ScanParams &p, hipStream_t st) {
    if (bf16) {
        if (ts.mode == kTileVec) return scan_bf16_vec_launch(output, ts, p, st);
        if (ts.mode == kTileMimo) return scan_bf16_mimo_launch(output, ts, p, st);
        return scan_bf16_gen_launch(output, ts, p, st);
    }
    return ts.mode == kTileVec ? scan_f32_vec_launch(output, ts, p, st) : scan_f32_gen_launch(output, ts, p, st);
}

hipError_t launch_seg_state(bool bf16, const TileShape &ts, const ScanParams &p, hipStream_t st) {
    return launch(false, bf16, ts, p, st);
}

hipError_t launch_seg_prefix(const TileShape &ts, const ScanParams &p, hipStream_t st) {
    const int per_q = ts.np * ts.pp / 4;
    const int64_t nwg = p.B * p.H * (int64_t)p.ncg * ((per_q + 255) / 256);
    if (nwg <= 0) return hipSuccess;
    hipLaunchKernelGGL(seg_prefix_kernel, dim3((unsigned)nwg), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_seg_output(bool bf16, const TileShape &ts, const ScanParams &p, hipStream_t st) {
    return launch(true, bf16, ts, p, st);
}

}  // namespace m3
