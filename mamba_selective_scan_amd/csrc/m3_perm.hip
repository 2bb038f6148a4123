// m3_perm.hip -- the N-axis permutation behind the half-split rotation pairing.
//
// The kernels rotate components (2i, 2i + 1) as pair i.  With the half-split pairing
// (pair i = components i and i + N/2) the computation is the same on the N axis
// permuted: user component i + c N/2 sits at kernel position 2 i + c.  The norm over N
// is permutation-invariant, and every other N-indexed quantity (gains, biases, the rows
// of the state and of prev_B) is permuted alongside.
#include "m3_internal.hpp"

namespace m3 {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void perm_n_kernel(const T *in, T *out, int64_t total, int N, int inner,
                                                     int to_kernel) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const int64_t row = e / inner;
    const int k = (int)(e - row * inner);
    const int64_t o = row / N;
    const int n = (int)(row - o * N), half = N / 2;
    int m;
    if (to_kernel) m = n < half ? 2 * n : 2 * (n - half) + 1;  // half-split n -> adjacent m
    else m = (n & 1) ? half + (n >> 1) : (n >> 1);             // adjacent n -> half-split m
    out[(o * N + m) * inner + k] = in[e];
}

// inner == 1 and N a multiple of 8: each thread moves 4 pairs (components i .. i+3 of both
// halves <-> adjacent positions 2i .. 2i+7) with 4-element vector loads and stores
template <typename T, typename V4>
__global__ __launch_bounds__(256) void perm_n4_kernel(const T *in, T *out, int64_t groups, int N, int to_kernel) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= groups) return;
    const int gpr = N / 8;  // groups of 4 pairs per row
    const int64_t o = e / gpr;
    const int j = (int)(e - o * gpr), half = N / 2;
    const T *src = in + o * N;
    T *dst = out + o * N;
    if (to_kernel) {
        const V4 a = *reinterpret_cast<const V4 *>(src + 4 * j), b = *reinterpret_cast<const V4 *>(src + half + 4 * j);
        const T *pa = reinterpret_cast<const T *>(&a), *pb = reinterpret_cast<const T *>(&b);
        V4 lo, hi;
        T *pl = reinterpret_cast<T *>(&lo), *ph = reinterpret_cast<T *>(&hi);
        pl[0] = pa[0]; pl[1] = pb[0]; pl[2] = pa[1]; pl[3] = pb[1];
        ph[0] = pa[2]; ph[1] = pb[2]; ph[2] = pa[3]; ph[3] = pb[3];
        *reinterpret_cast<V4 *>(dst + 8 * j) = lo;
        *reinterpret_cast<V4 *>(dst + 8 * j + 4) = hi;
    } else {
        const V4 lo = *reinterpret_cast<const V4 *>(src + 8 * j), hi = *reinterpret_cast<const V4 *>(src + 8 * j + 4);
        const T *pl = reinterpret_cast<const T *>(&lo), *ph = reinterpret_cast<const T *>(&hi);
        V4 a, b;
        T *pa = reinterpret_cast<T *>(&a), *pb = reinterpret_cast<T *>(&b);
        pa[0] = pl[0]; pb[0] = pl[1]; pa[1] = pl[2]; pb[1] = pl[3];
        pa[2] = ph[0]; pb[2] = ph[1]; pa[3] = ph[2]; pb[3] = ph[3];
        *reinterpret_cast<V4 *>(dst + 4 * j) = a;
        *reinterpret_cast<V4 *>(dst + half + 4 * j) = b;
    }
}

}  // namespace

hipError_t launch_perm_n(const void *in, void *out, int64_t outer, int N, int inner, int esize, bool to_kernel,
                         hipStream_t stream) {
    const int64_t total = outer * N * (int64_t)inner;
    if (total <= 0) return hipSuccess;
    if (inner == 1 && N % 8 == 0) {
        const int64_t groups = outer * (N / 8);
        const dim3 g4((unsigned)((groups + 255) / 256));
        if (esize == 2)
            hipLaunchKernelGGL((perm_n4_kernel<uint16_t, uint2>), g4, dim3(256), 0, stream, (const uint16_t *)in,
                               (uint16_t *)out, groups, N, to_kernel ? 1 : 0);
        else
            hipLaunchKernelGGL((perm_n4_kernel<uint32_t, uint4>), g4, dim3(256), 0, stream, (const uint32_t *)in,
                               (uint32_t *)out, groups, N, to_kernel ? 1 : 0);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((total + 255) / 256));
    if (esize == 2)
        hipLaunchKernelGGL(perm_n_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t *)in,
                           (uint16_t *)out, total, N, inner, to_kernel ? 1 : 0);
    else
        hipLaunchKernelGGL(perm_n_kernel<uint32_t>, grid, dim3(256), 0, stream, (const uint32_t *)in,
                           (uint32_t *)out, total, N, inner, to_kernel ? 1 : 0);
    return hipGetLastError();
}

}  // namespace m3
