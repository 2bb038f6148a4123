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

}  // namespace

hipError_t launch_perm_n(const void *in, void *out, int64_t outer, int N, int inner, int esize, bool to_kernel,
                         hipStream_t stream) {
    const int64_t total = outer * N * (int64_t)inner;
    if (total <= 0) return hipSuccess;
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
