// 8-bit expert weights: OCP E4M3 codes with one fp32 scale per row.
//
// youleyou.com article, "Deployment": the model ships tuned for a 4-bit
// floating-point weight format on NVIDIA parts, so the memory-bound experts
// move fewer bytes.  The CDNA4 analogue is OCP E4M3 ("e4m3fn": 1 sign, 4
// exponent bits with bias 7, 3 mantissa bits, largest finite 448, no
// infinity), which gfx950 decodes in hardware (v_cvt_pk_f32_fp8).
//
// Per row: amax = max |x|, scale = amax / 448 in binary32 (1 when amax = 0),
// code = E4M3 of the binary32 quotient x / scale, round to nearest with
// ties to the even code, magnitudes at or above 448 giving 448.
#include "common.h"
#include "kernels.h"

namespace dg {

namespace {

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

// One workgroup per row: the row's amax, then four codes per thread step.
template <typename T>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T* __restrict__ src, int cols,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scale) {
    const long row = blockIdx.x;
    const T* x = src + row * cols;
    float amax = 0.0f;
    for (int i = threadIdx.x; i < cols; i += 256) amax = fmaxf(amax, fabsf(Elt<T>::to_f(x[i])));
    amax = wave_max(amax);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    if (threadIdx.x == 0) scale[row] = s;
    uint8_t* out = q + row * cols;
    for (int i = threadIdx.x; i < cols; i += 256) out[i] = (uint8_t)e4m3_code(Elt<T>::to_f(x[i]) / s);
}

}  // namespace

template <typename T>
hipError_t quantize_fp8(const T* src, long rows, int cols, uint8_t* q, float* scale,
                        hipStream_t st) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    if (rows > 0x7FFFFFFFL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_fp8_kernel<T>, dim3((unsigned)rows), dim3(256), 0, st, src, cols, q,
                       scale);
    return hipGetLastError();
}

template hipError_t quantize_fp8<float>(const float*, long, int, uint8_t*, float*, hipStream_t);
template hipError_t quantize_fp8<bf16_t>(const bf16_t*, long, int, uint8_t*, float*, hipStream_t);

}  // namespace dg
