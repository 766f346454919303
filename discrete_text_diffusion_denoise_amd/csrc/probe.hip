// Microbenchmark peaks of the GPU the library runs on, reported beside the
// published ones by the benchmark: a read-only HBM stream and a loop of
// independent bf16 MFMAs.  Measurement aids only; no step of the denoising
// path calls them.
#include <hip/hip_runtime.h>

#include "dg.h"
#include "kernels.h"

namespace dg {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Every thread streams 16-byte pieces of the buffer (grid-stride, four
// loads in flight) and folds them into one word, written per thread so that
// no load is dead.  out holds one word per launched thread.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* __restrict__ src, long n,
                                                         uint32_t* __restrict__ out) {
    const long stride = (long)gridDim.x * 256;
    long i = (long)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
        const u32x4_t v = (a ^ b) + (c ^ d);
        acc ^= (v.x ^ v.y) + (v.z ^ v.w);
    }
    for (; i < n; i += stride) acc ^= src[i].x;
    out[(long)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Four independent 16x16x32 bf16 MFMA accumulators per wave, `iters` rounds.
// The MFMAs are one asm block per round so that the compiler keeps the
// accumulators in place (written as builtins in a loop, it rotates them
// through register moves).  The result goes to out, one word per thread.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float seed, float* out) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
        b[i] = (__bf16)(seed * (float)(i + 1));
    }
    f32x4_t c0 = {seed, 0.f, 0.f, 0.f}, c1 = {2.f * seed, 0.f, 0.f, 0.f};
    f32x4_t c2 = {3.f * seed, 0.f, 0.f, 0.f}, c3 = {4.f * seed, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
        asm volatile(
            "v_mfma_f32_16x16x32_bf16 %0, %4, %5, %0\n v_mfma_f32_16x16x32_bf16 %1, %4, %5, %1\n"
            "v_mfma_f32_16x16x32_bf16 %2, %4, %5, %2\n v_mfma_f32_16x16x32_bf16 %3, %4, %5, %3"
            : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
            : "v"(a), "v"(b));
    }
    // the last MFMA results must be complete before a VALU reads them
    asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
    const f32x4_t t = c0 + c1 + c2 + c3;
    out[(long)blockIdx.x * 256 + threadIdx.x] = t[0] + t[1] + t[2] + t[3];
}

}  // namespace

}  // namespace dg

extern "C" dg_status dg_measure_peaks(void* d_buf, size_t buf_bytes, void* stream,
                                      double* hbm_read_gbs, double* mfma_bf16_tflops) {
    using namespace dg;
    if (!d_buf || !hbm_read_gbs || !mfma_bf16_tflops) return DG_ERR_ARG;
    const int cus = cu_count();
    const long out_words = (long)cus * 8 * 256;   // the larger of the two grids' thread counts
    if (cus <= 0 || buf_bytes < (size_t)(256u << 20) + (size_t)out_words * 4) return DG_ERR_CAPACITY;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // the read stream covers the buffer after the output words, in 16-byte pieces
    char* base = static_cast<char*>(d_buf);
    uint32_t* out = reinterpret_cast<uint32_t*>(base);
    const size_t off = ((size_t)out_words * 4 + 4095) & ~(size_t)4095;
    const long n = (long)((buf_bytes - off) / 16);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(base + off);
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return DG_ERR_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return DG_ERR_HIP;
    }
    dg_status rc = DG_OK;
    float ms = 0.f;
    const int reps = 5;
    // read: 8 workgroups of 256 threads a CU, the first pass untimed
    hipLaunchKernelGGL(read_probe_kernel, dim3(cus * 8), dim3(256), 0, st, src, n, out);
    (void)hipEventRecord(e0, st);
    for (int r = 0; r < reps; ++r)
        hipLaunchKernelGGL(read_probe_kernel, dim3(cus * 8), dim3(256), 0, st, src, n, out);
    (void)hipEventRecord(e1, st);
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f) {
        rc = DG_ERR_HIP;
    } else {
        *hbm_read_gbs = (double)n * 16.0 * reps / (ms * 1e-3) / 1e9;
    }
    // MFMA: eight waves a SIMD (8 workgroups of 4 waves a CU), 4 x iters MFMAs a wave
    const int iters = 20000;
    float* fout = reinterpret_cast<float*>(base);
    if (rc == DG_OK) {
        hipLaunchKernelGGL(mfma_probe_kernel, dim3(cus * 8), dim3(256), 0, st, 100, 1e-3f, fout);
        (void)hipEventRecord(e0, st);
        hipLaunchKernelGGL(mfma_probe_kernel, dim3(cus * 8), dim3(256), 0, st, iters, 1e-3f, fout);
        (void)hipEventRecord(e1, st);
        if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f) {
            rc = DG_ERR_HIP;
        } else {
            const double flop = (double)cus * 8 * 4 * (double)iters * 4 * 16.0 * 16.0 * 32.0 * 2.0;
            *mfma_bf16_tflops = flop / (ms * 1e-3) / 1e12;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return rc;
}
