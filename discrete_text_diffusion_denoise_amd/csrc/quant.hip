// Low-precision expert weights: OCP E4M3 codes with one fp32 scale per row,
// and OCP MXFP4 (E2M1 codes with an E8M0 scale per 32 elements).
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
#include "mx.h"

namespace dg {

namespace {

// Tiled layout of the codes (the block-scaled expert kernels' operand order):
// 16-row tiles, each a run of 128-column steps; a tile-step is two 1-KiB
// halves (columns 0..63 and 64..127 of the step), and in half h the 16-byte
// chunk 16 g + r holds row r's columns 64 h + 16 g .. +15.
__device__ __forceinline__ long fp8_tiled_index(long row, int col, int cols) {
    const long tile = row >> 4;
    const int r = (int)(row & 15), s = col >> 7, kk = col & 127;
    const int h = kk >> 6, g = (kk >> 4) & 3, p = kk & 15;
    return ((tile * (cols >> 7) + s) * 2 + h) * 1024 + (16 * g + r) * 16 + p;
}

// One workgroup per row: the row's amax, then one code per thread step.
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
    for (int i = threadIdx.x; i < cols; i += 256)
        q[fp8_tiled_index(row, i, cols)] = (uint8_t)e4m3_code(Elt<T>::to_f(x[i]) / s);
}

// ------------------------------------------------------------------ MXFP4
// OCP microscaling: 32 consecutive elements of a row share an E8M0 scale
// X = 2^(floor(log2(max |v|)) - 2) (2 = the exponent of E2M1's largest value
// 6), clamped to 2^-127 .. 2^127 (an all-zero block takes 2^-127); each
// element is v / X rounded to the nearest E2M1 value (0, 0.5, 1, 1.5, 2, 3,
// 4, 6; ties to the even code), magnitudes above 6 giving 6.

// E2M1 code of a finite binary32 value (sign kept): the round-to-nearest
// thresholds are the midpoints of the value table, a midpoint going to the
// neighbour with the even code.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
    const float a = fabsf(v);
    uint32_t c;
    if (a <= 0.25f) c = 0;            // 0.25: 0 (code 0) against 0.5 (code 1)
    else if (a < 0.75f) c = 1;        // 0.75: 1.0 (code 2)
    else if (a <= 1.25f) c = 2;       // 1.25: 1.0 (code 2) against 1.5
    else if (a < 1.75f) c = 3;        // 1.75: 2.0 (code 4)
    else if (a <= 2.5f) c = 4;        // 2.5: 2.0 (code 4) against 3.0
    else if (a < 3.5f) c = 5;         // 3.5: 4.0 (code 6)
    else if (a <= 5.0f) c = 6;        // 5.0: 4.0 (code 6) against 6.0
    else c = 7;
    return sign | c;
}

// One thread per 32-element block: the block's scale code, then its 16
// bytes of codes (two per byte, the even element in the low nibble).  Tiled
// layout (the block-scaled expert kernels' operand order): 16-row tiles, each
// a run of 128-column steps; in a tile-step the 16 code bytes of block g of
// row r are chunk 16 g + r of 1 KiB, and its scale code is byte 16 g + r of
// 64.
template <typename T>
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const T* __restrict__ src, long rows,
                                                             int cols, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ scale) {
    const int nb = cols / 32;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * nb) return;
    const long row = idx / nb;
    const int b = (int)(idx % nb);
    const T* x = src + row * cols + (long)b * 32;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        v[i] = Elt<T>::to_f(x[i]);
        amax = fmaxf(amax, fabsf(v[i]));
    }
    int ex = -127;
    if (amax > 0.0f) {
        int e2;
        (void)frexpf(amax, &e2);            // amax = m 2^e2, m in [0.5, 1)
        ex = e2 - 1 - 2;
        ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
    }
    const float inv = ldexpf(1.0f, -ex);    // exact: a power of two
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i >> 3] |= e2m1_code(v[i] * inv) << (4 * (i & 7));
    const long ts = (row >> 4) * (cols >> 7) + (b >> 2);        // tile-step
    const int lane = 16 * (b & 3) + (int)(row & 15);
    *reinterpret_cast<uint4*>(q + ts * 1024 + lane * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    scale[ts * 64 + lane] = (uint8_t)(ex + 127);
}

}  // namespace

template <typename T>
hipError_t quantize_mxfp4(const T* src, long rows, int cols, uint8_t* q, uint8_t* scale,
                          hipStream_t st) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    if (cols % 128 || rows % 16) return hipErrorInvalidValue;
    const long blocks = rows * (cols / 32);
    if (blocks / 256 + 1 > 0x7FFFFFFFL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_mxfp4_kernel<T>, dim3((unsigned)((blocks + 255) / 256)), dim3(256),
                       0, st, src, rows, cols, q, scale);
    return hipGetLastError();
}

template hipError_t quantize_mxfp4<float>(const float*, long, int, uint8_t*, uint8_t*, hipStream_t);
template hipError_t quantize_mxfp4<bf16_t>(const bf16_t*, long, int, uint8_t*, uint8_t*,
                                           hipStream_t);

template <typename T>
hipError_t quantize_fp8(const T* src, long rows, int cols, uint8_t* q, float* scale,
                        hipStream_t st) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    if (rows > 0x7FFFFFFFL || cols % 128 || rows % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_fp8_kernel<T>, dim3((unsigned)rows), dim3(256), 0, st, src, cols, q,
                       scale);
    return hipGetLastError();
}

template hipError_t quantize_fp8<float>(const float*, long, int, uint8_t*, float*, hipStream_t);
template hipError_t quantize_fp8<bf16_t>(const bf16_t*, long, int, uint8_t*, float*, hipStream_t);

}  // namespace dg
