// Device-side building blocks shared by the retention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "retention.h"

namespace ret {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxHeads = RETENTION_MAX_HEADS;
constexpr int kMaxPairs = RETENTION_MAX_DK / 2;

// Per-call scalars that every kernel needs. Travels by value in the kernel
// arguments; gamma and theta are copied from the caller's host arrays.
struct HeadParams {
    float gamma[kMaxHeads];
    float theta[kMaxPairs];
    int has_theta;
};

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_to_f32(u16 h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 packed in 32 bits (low half = lo), rounded to
// nearest even by gfx950's v_cvt_pk_bf16_f32; NaN stays NaN.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- MFMA

// D = A(16x32) * B(32x16) + C on bf16 operands with float32 accumulation.
// Lane l supplies row/column (l % 16) and the 8 contraction indices of group
// (l / 16); the accumulator holds rows 4*(l/16) + r, column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(const uint4& a, const uint4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- decay

// log2(gamma) and gamma^n for this head, formed in float64 so that heads with
// gamma close to 1 keep their precision.
__device__ __forceinline__ double log2_gamma(float g) { return log2(static_cast<double>(g)); }

__device__ __forceinline__ float gamma_pow(double lg2, double n) {
    return static_cast<float>(exp2(lg2 * n));
}

// 2^x on the hardware transcendental unit (one instruction; results below
// the float32 normal range flush toward zero, which only affects decay
// factors far below any retained contribution).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- rotation

// cos/sin of position * theta with the product and the reduction to
// [-pi, pi] done in float64, then float32 sin/cos of the reduced angle.
__device__ __forceinline__ void rot_cs(double position, float theta, float& c, float& s) {
    const double two_pi = 6.283185307179586476925286766559;
    double a = position * static_cast<double>(theta);
    a -= two_pi * rint(a / two_pi);
    sincosf(static_cast<float>(a), &s, &c);
}

// cos/sin of position * theta for operands that are rounded to bf16 next:
// the angle in revolutions is formed and reduced to [-1/2, 1/2] in float64,
// then the hardware sin/cos (which take revolutions) evaluate it. Their
// absolute error is far below bf16 resolution, and the code stays small
// enough to unroll around MFMA operand registers.
__device__ __forceinline__ void rot_cs_fast(double position, float theta, float& c, float& s) {
    const double inv_two_pi = 0.15915494309189533576888376337251;
    double rev = position * (static_cast<double>(theta) * inv_two_pi);
    rev -= rint(rev);
    const float r = static_cast<float>(rev);
    s = __builtin_amdgcn_sinf(r);
    c = __builtin_amdgcn_cosf(r);
}

// Rotate the four complex pairs held in 8 consecutive bf16 (one uint4) with
// frequencies th[0..3], at absolute position `position`.
__device__ __forceinline__ uint4 rotate8_bf16(uint4 x, const float* th, double position) {
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float c, s;
        rot_cs_fast(position, th[p], c, s);
        float re = lo_bf16(w[p]), im = hi_bf16(w[p]);
        w[p] = pack2_bf16(re * c - im * s, re * s + im * c);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// The same with the frequencies of pairs j0..j0+3 read from the head parameters.
__device__ __forceinline__ uint4 rotate8_bf16(uint4 x, const HeadParams& hp, int j0, double position) {
    return rotate8_bf16(x, hp.theta + j0, position);
}

// ---------------------------------------------------------------- launch grid

// The 8 XCDs of the MI355X take workgroups round-robin by id. Re-number so
// that consecutive logical ids run on the same XCD (and share its L2), which
// keeps the value tiles of one head together. Identity when the grid is not a
// multiple of 8.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
    if ((nblocks & 7) != 0) return bid;
    return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

}  // namespace ret
