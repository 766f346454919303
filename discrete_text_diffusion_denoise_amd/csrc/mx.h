// OCP 8-bit floating point (E4M3) encoding and the MXFP8 shared scale, used
// by the weight quantiser, by the normalisation that feeds the experts and by
// the expert kernels' epilogue.
//
// E4M3 ("e4m3fn"): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
// largest finite value 448, no infinity.  MXFP8 (OCP microscaling v1.0):
// 32 consecutive elements share the E8M0 scale X = 2^(floor(log2(max |v|))
// - 8), 8 being the exponent of 448; clamped to 2^-127 .. 2^127, an all-zero
// block taking 2^-127; each element is the E4M3 code of v / X.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// E4M3 code of a finite binary32 value: sign kept; below 2^-6 the
// subnormal steps of 2^-9 (round half to even on the step count, 8 steps
// being the smallest normal code 0x08); above, the binary32 mantissa rounded
// to 3 bits (half to even, a carry moving into the exponent); saturating at
// 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    uint32_t c;
    if (!(a < 448.0f)) {
        c = 0x7Eu;
    } else if (a < 0.015625f) {
        c = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        const uint32_t b = __float_as_uint(a);
        const uint32_t e = (b >> 23) - 127u + 7u;     // 1 .. 15
        const uint32_t m = b & 0x7FFFFFu;
        c = (e << 3) | (m >> 20);
        const uint32_t rem = m & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (c & 1u))) c += 1u;
        c = c > 0x7Eu ? 0x7Eu : c;
    }
    return sign | c;
}

// Activation code: e4m3_code, except that a NaN or infinite value gives the
// NaN code 0x7F, so a non-finite activation stays visible in the product.
__device__ __forceinline__ uint32_t e4m3_act(float v) {
    return (v - v == 0.0f) ? e4m3_code(v) : 0x7Fu;
}

// Exponent of the MXFP8 shared scale of a block with largest magnitude amax
// (finite, >= 0): floor(log2(amax)) - 8, clamped to [-127, 127]; -127 for 0.
__device__ __forceinline__ int mx8_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    int e2;
    (void)frexpf(amax, &e2);            // amax = m 2^e2, m in [0.5, 1)
    const int ex = e2 - 1 - 8;
    return ex < -127 ? -127 : (ex > 127 ? 127 : ex);
}

}  // namespace dg
