// m3_device.hpp -- device-side helpers for the gfx950 Mamba-3 kernels:
// bf16 rounding, hi/lo operand splitting, MFMA wrappers, angle reduction.
//
// Matrix-core conventions used everywhere (checked on gfx950 hardware):
//   v_mfma_f32_16x16x32_bf16: lane l, slot j (0..7) of A holds A[l%16][8*(l/16)+j],
//     slot j of B holds B[8*(l/16)+j][l%16]; result slot i (0..3) is C[4*(l/16)+i][l%16].
//   v_mfma_f32_16x16x4_f32:  lane l of A holds A[l%16][l/16], of B holds B[l/16][l%16].
// A "fragment" here is 8 values per lane along the contraction index k; the
// only requirement is that A and B agree on which logical k each (lane group,
// slot) carries.  For the fp32 path a fragment feeds 8 consecutive 16x16x4
// MFMAs (slot j -> instruction j).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Debug builds (-DM3_DEBUG): device-side bounds and plan checks.  A failed check does not
// trap: it counts itself and records its source line in two words that the host reads back
// (m3_debug_checks), so a bad index is reported without faulting the device.  Release builds
// compile the checks out.
#ifdef M3_DEBUG
#define M3_DCHECK(p, cond)                                   \
    do {                                                     \
        if (!(cond) && (p).dbg) {                            \
            atomicAdd((p).dbg, 1u);                          \
            atomicMax((p).dbg + 1, (unsigned int)__LINE__);  \
        }                                                    \
    } while (0)
#else
#define M3_DCHECK(p, cond) \
    do {                   \
    } while (0)
#endif

namespace m3 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ uint32_t f2bf(float f) {  // round to nearest, ties to even
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// split v into hi + lo, both bf16 (hi = rne(v), lo = rne(v - hi)); |v - hi - lo| <= 2^-17 |v|
__device__ __forceinline__ void split_hl(float v, uint32_t &hi, uint32_t &lo) {
    hi = f2bf(v);
    lo = f2bf(v - bf2f(hi));
}
__device__ __forceinline__ uint32_t pack2(uint32_t a, uint32_t b) { return a | (b << 16); }

// ---------------------------------------------------------------- io types
struct IoF32 {
    typedef float T;
    static constexpr int bytes = 4;
    __device__ __forceinline__ static float ld(const float *p) { return *p; }
    __device__ __forceinline__ static void st(float *p, float v) { *p = v; }
};
struct IoBF16 {
    typedef uint16_t T;
    static constexpr int bytes = 2;
    __device__ __forceinline__ static float ld(const uint16_t *p) { return bf2f(*p); }
    __device__ __forceinline__ static void st(uint16_t *p, float v) { *p = (uint16_t)f2bf(v); }
};

// ---------------------------------------------------------------- operand fragments
// Hi/lo bf16 operand (3-product emulation of an fp32 operand) or an fp32 operand.
struct FragHL { u32x4_t hi, lo; };
struct FragF { float v[8]; };

__device__ __forceinline__ f32x4_t mfma_bf(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A * B, both split:  hi*hi + hi*lo + lo*hi  (the lo*lo term is below fp32 rounding of the sum)
__device__ __forceinline__ f32x4_t mma(const FragHL &a, const FragHL &b, f32x4_t c) {
    c = mfma_bf(a.lo, b.hi, c);
    c = mfma_bf(a.hi, b.lo, c);
    c = mfma_bf(a.hi, b.hi, c);
    return c;
}
// acc += A * B with B exact in bf16
__device__ __forceinline__ f32x4_t mma(const FragHL &a, const u32x4_t &b, f32x4_t c) {
    c = mfma_bf(a.lo, b, c);
    c = mfma_bf(a.hi, b, c);
    return c;
}
__device__ __forceinline__ f32x4_t mma(const u32x4_t &a, const FragHL &b, f32x4_t c) {
    c = mfma_bf(a, b.lo, c);
    c = mfma_bf(a, b.hi, c);
    return c;
}
__device__ __forceinline__ f32x4_t mma(const FragF &a, const FragF &b, f32x4_t c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = mfma_f(a.v[j], b.v[j], c);
    return c;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- fp16 operands
// A single fp16 operand (8 halves per lane, same lane layout as the bf16 MFMA).  Used for the
// normalised, rotated B~ and C~ and for the carried state H, each held within the fp16 range
// by a power-of-two scale that the caller undoes after the product (scales are exact).
struct FragH { u32x4_t v; };
__device__ __forceinline__ f32x4_t mfma_h(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                  c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma(const FragH &a, const FragH &b, f32x4_t c) { return mfma_h(a.v, b.v, c); }
// two floats -> packed fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}
// acc + the squares of the two bf16 halves of w (one v_dot2 instruction)
__device__ __forceinline__ float sumsq2_bf16(uint32_t w, float acc) {
    const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}
// 2^(k - e) and 2^(e - k) for the exponent e of m (m = f 2^e, f in [0.5, 1)): a power of two
// that maps m into [2^(k-1), 2^k), and its inverse; (1, 1) for m == 0 or a non-finite m
template <int K>
__device__ __forceinline__ void pow2_scale(float m, float &s, float &inv) {
    const int e = __builtin_amdgcn_frexp_expf(m);
    const bool ok = m > 0.f && m < 3.0e38f;
    s = ok ? __builtin_ldexpf(1.f, K - e) : 1.f;
    inv = ok ? __builtin_ldexpf(1.f, e - K) : 1.f;
}

// two floats -> packed bf16 words hi = rne(v), lo = rne(v - hi) (one v_cvt_pk_bf16_f32 each)
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    const uint32_t hu = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
    const float ha = __uint_as_float(hu << 16), hb = __uint_as_float(hu & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a - ha, b - hb}, bf16x2_t));
    hi = hu;
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// build a hi/lo fragment from 8 floats
__device__ __forceinline__ FragHL make_hl(const float (&v)[8]) {
    FragHL f;
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split2(v[2 * j], v[2 * j + 1], h[j], l[j]);
    f.hi = u32x4_t{h[0], h[1], h[2], h[3]};
    f.lo = u32x4_t{l[0], l[1], l[2], l[3]};
    return f;
}
__device__ __forceinline__ FragF make_f(const float (&v)[8]) {
    FragF f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = v[j];
    return f;
}

// ---------------------------------------------------------------- angles
// Reduce an angle to [0, 2 pi) in double precision (exact enough for any float input).
__device__ __forceinline__ double wrap_2pi(double a) {
    const double two_pi = 6.283185307179586476925286766559;
    const double inv_two_pi = 0.15915494309189533576888376337251;
    double k = floor(a * inv_two_pi);
    double r = a - k * two_pi;
    if (r < 0.0) r += two_pi;
    if (r >= two_pi) r -= two_pi;
    return r;
}

// sin and cos of an angle with the hardware sin/cos units, which take the
// argument in revolutions: the angle is scaled by 1 / (2 pi) and its fractional
// part taken.  The scaling rounds to 2^-24 of the angle, below the float
// resolution of the angle itself; callers pass block-local running sums or
// angles already reduced to [0, 2 pi).
__device__ __forceinline__ void fast_sincos(float a, float &s, float &c) {
    const float rev = __builtin_amdgcn_fractf(a * 0.15915494309189535f);
    s = __builtin_amdgcn_sinf(rev);
    c = __builtin_amdgcn_cosf(rev);
}
__device__ __forceinline__ f32x2_t sincos_acc(float a) {
    float s, c;
    fast_sincos(a, s, c);
    return f32x2_t{s, c};
}

// ---------------------------------------------------------------- cross-lane scans and reductions
// v + (value of the lane K to the left inside its row of 16 lanes, or 0)
template <int K>
__device__ __forceinline__ float add_row_shr(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + K, 0xF, 0xF, true));
}
// inclusive add-scan over the 16 lanes of each DPP row
__device__ __forceinline__ float row_incl_scan(float v) {
    v = add_row_shr<1>(v);
    v = add_row_shr<2>(v);
    v = add_row_shr<4>(v);
    v = add_row_shr<8>(v);
    return v;
}

// inclusive add-scan of 64 lanes (every lane of the wave must be active): scans
// inside the rows of 16, then row 0's total is broadcast into row 1 (and row 2's
// into row 3), then row 1's running total into rows 2 and 3
__device__ __forceinline__ float wave_incl_scan(float v) {
    v = row_incl_scan(v);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return v;
}

// Sum and maximum over the four 16-lane rows of a wave, returned to every lane.  With both
// operands the same value, permlane16_swap hands each lane the value of the same lane in the
// neighbouring row (rows 0-1, 2-3) and permlane32_swap that of the other half: the xor-16 /
// xor-32 butterfly in two VALU exchanges instead of two LDS permutes, with the same bits (each
// step adds or compares the same two values on both lanes of a pair).
__device__ __forceinline__ float rows_sum4(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max4(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ---------------------------------------------------------------- block activations
// Input activations of the canonical block: dt = softplus(raw + bias) in the
// overflow-safe form max(v, 0) + log1p(exp(-|v|)); lambda = sigmoid(raw) (reciprocal
// to 1 ulp; exp overflow at raw << 0 gives 0, the limit).
__device__ __forceinline__ float softplus_f(float v) { return fmaxf(v, 0.f) + log1pf(__expf(-fabsf(v))); }
__device__ __forceinline__ float sigmoid_f(float v) { return __builtin_amdgcn_rcpf(1.f + __expf(-v)); }
// Output gate silu(z) = z sigmoid(z) (exp overflow at z << 0 gives -0, the limit).
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

}  // namespace m3
