// Bandwidth-bound helpers of the step: RMSNorm, embedding gather, split-K
// reduction, transpose, and RoPE with the KV-cache write.
#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace dg {

namespace {

// The outputs of a normalised float4 r at column i of row `row`: u (T),
// optionally u32 (fp32) and the MXFP8 codes q8 / scale codes q8s (d % 32 == 0;
// a 32-column block is the float4s of 8 consecutive threads).
template <typename T>
__device__ __forceinline__ void rms_write(const float4 r, long row, int i, int d, T* o,
                                          float* __restrict__ u32, uint8_t* __restrict__ q8,
                                          uint8_t* __restrict__ q8s) {
    o[i + 0] = Elt<T>::from_f(r.x);
    o[i + 1] = Elt<T>::from_f(r.y);
    o[i + 2] = Elt<T>::from_f(r.z);
    o[i + 3] = Elt<T>::from_f(r.w);
    if (u32) *reinterpret_cast<float4*>(u32 + row * d + i) = r;
    if (q8) {
        // the 8 threads of a block hold the same loop trip count (d % 32 == 0)
        float m = fmaxf(fmaxf(fabsf(r.x), fabsf(r.y)), fmaxf(fabsf(r.z), fabsf(r.w)));
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        const int ex = mx8_exponent(m);
        const float inv = __builtin_amdgcn_ldexpf(1.0f, -ex);   // exact: a power of two
        const uint32_t code = e4m3_act(r.x * inv) | (e4m3_act(r.y * inv) << 8) |
                              (e4m3_act(r.z * inv) << 16) | (e4m3_act(r.w * inv) << 24);
        *reinterpret_cast<uint32_t*>(q8 + row * d + i) = code;
        if ((threadIdx.x & 7) == 0) q8s[row * (d / 32) + i / 32] = (uint8_t)(ex + 127);
    }
}

// One workgroup per row: sum of squares in fp32, then scale.  With q8 set,
// the fp32 result is also written as MXFP8 (d % 32 == 0): E4M3 codes into
// q8 [rows][d] and the E8M0 scale code of each 32-element block into q8s
// [rows][d / 32]; a block is the 4 values of 8 consecutive threads.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h,
                                                      const float* __restrict__ w,
                                                      T* __restrict__ u, int d, float eps,
                                                      float* __restrict__ u32,
                                                      uint8_t* __restrict__ q8,
                                                      uint8_t* __restrict__ q8s) {
    const long row = blockIdx.x;
    const float* x = h + row * d;
    float ss = 0.f;
    for (int i = threadIdx.x * 4; i < d; i += 256 * 4)
        ss = rms_accum(ss, *reinterpret_cast<const float4*>(x + i));
    __shared__ float part[4];
    const float scale = rms_block_scale(ss, part, d, eps);
    T* o = u + row * d;
    for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
        const float4 r = rms_apply(*reinterpret_cast<const float4*>(x + i), scale, w, i);
        rms_write(r, row, i, d, o, u32, q8, q8s);
    }
}


// The residual add of a split-K product (h += sum over the splits of part
// [splits][rows][d], in split order) with the RMSNorm of the new rows fused:
// one workgroup a row in rmsnorm_kernel's layout, the same outputs and bits
// as splitk_epilogue (EPI_ADD_F32) followed by rmsnorm.
template <typename T>
__global__ __launch_bounds__(256) void splitk_add_norm_kernel(const float* __restrict__ part,
                                                              int splits, long rows,
                                                              float* __restrict__ h,
                                                              const float* __restrict__ w,
                                                              T* __restrict__ u, int d, float eps,
                                                              float* __restrict__ u32,
                                                              uint8_t* __restrict__ q8,
                                                              uint8_t* __restrict__ q8s) {
    const long row = blockIdx.x;
    float* x = h + row * d;
    const float* pr = part + row * d;
    const long zs = rows * d;
    float ss = 0.f;
    for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
        const float4 v = splitk_sum4(pr + i, zs, splits);
        float4 hv = *reinterpret_cast<const float4*>(x + i);
        hv.x = hv.x + v.x;
        hv.y = hv.y + v.y;
        hv.z = hv.z + v.z;
        hv.w = hv.w + v.w;
        *reinterpret_cast<float4*>(x + i) = hv;
        ss = rms_accum(ss, hv);
    }
    __shared__ float pt[4];
    const float scale = rms_block_scale(ss, pt, d, eps);
    T* o = u + row * d;
    for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
        const float4 r = rms_apply(*reinterpret_cast<const float4*>(x + i), scale, w, i);
        rms_write(r, row, i, d, o, u32, q8, q8s);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ E,
                                                    const int32_t* __restrict__ tok, int ld,
                                                    int n, int V, float* __restrict__ h, int d) {
    const long row = blockIdx.x;   // b*n + i
    const long b = row / n, i = row % n;
    const int id = min(max(tok[b * ld + i], 0), V - 1);   // ids outside [0, V) never index past E
    const T* e = E + (long)id * d;
    float* o = h + row * d;
    // eight loads in flight before their stores
    int k = threadIdx.x;
    for (; k + 7 * 256 < d; k += 8 * 256) {
        T v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = e[k + q * 256];
#pragma unroll
        for (int q = 0; q < 8; ++q) o[k + q * 256] = Elt<T>::to_f(v[q]);
    }
    for (; k < d; k += 256) o[k] = Elt<T>::to_f(e[k]);
}

template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            T* __restrict__ out, int splits,
                                                            long total, int cols,
                                                            const float* __restrict__ row_stats) {
    long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    // summed in split order, eight loads in flight before their adds
    float s = 0.f;
    int z = 0;
    for (; z + 8 <= splits; z += 8) {
        float p[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) p[q] = part[(long)(z + q) * total + i];
#pragma unroll
        for (int q = 0; q < 8; ++q) s += p[q];
    }
    for (; z < splits; ++z) s += part[(long)z * total + i];
    if (row_stats) s = s * (1.0f / row_stats[(i / cols) * 4 + 1]);
    out[i] = Elt<T>::from_f(s);
}

__global__ __launch_bounds__(256) void widen_kernel(const bf16_t* __restrict__ in,
                                                   float* __restrict__ out, long n) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = bf2f(in[i]);
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int32_t v, long n) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// Top-k self-conditioning: s[row] = sum_i p_i E[idx_i] over the row's K
// candidates, in candidate order (fp32).  A thread owns 8 consecutive
// columns (16 bytes of a bf16 row); the candidates' rows are loaded eight at
// a time, so eight loads per thread are in flight.
template <typename T>
__global__ __launch_bounds__(256) void selfcond_topk_kernel(const T* __restrict__ E, int d,
                                                            const int32_t* __restrict__ idx,
                                                            const float* __restrict__ p, int K,
                                                            T* __restrict__ out) {
    const long row = blockIdx.x;
    const int32_t* ri = idx + row * K;
    const float* rp = p + row * K;
    for (int c0 = threadIdx.x * 8; c0 < d; c0 += 256 * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int i0 = 0; i0 < K; i0 += 8) {
            float v[8][8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = min(i0 + u, K - 1);
                const T* src = E + (long)ri[i] * d + c0;
#pragma unroll
                for (int q = 0; q < 8; ++q) v[u][q] = Elt<T>::to_f(src[q]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (i0 + u < K) {
                    const float w = rp[i0 + u];
#pragma unroll
                    for (int q = 0; q < 8; ++q) acc[q] += w * v[u][q];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) out[row * d + c0 + q] = Elt<T>::from_f(acc[q]);
    }
}

// RMSNorm of fp32 rows into the blocked bf16 layout (rows padded to 256 are
// not written).
__global__ __launch_bounds__(256) void rmsnorm_tiled_kernel(const float* __restrict__ h,
                                                            const float* __restrict__ w,
                                                            bf16_t* __restrict__ u, int d,
                                                            float eps) {
    const long row = blockIdx.x;
    const float* x = h + row * d;
    float ss = 0.f;
    for (int i = threadIdx.x * 4; i < d; i += 256 * 4)
        ss = rms_accum(ss, *reinterpret_cast<const float4*>(x + i));
    __shared__ float part[4];
    const float scale = rms_block_scale(ss, part, d, eps);
    for (int i = threadIdx.x * 4; i < d; i += 256 * 4) {
        const float4 r = rms_apply(*reinterpret_cast<const float4*>(x + i), scale, w, i);
        *reinterpret_cast<uint2*>(u + tiled_index(row, i, d)) =
            make_uint2(pack_bf2(r.x, r.y), pack_bf2(r.z, r.w));
    }
}

// E [V][d] (bf16) into the blocked layout of E (rows V, padded with zeros to
// a multiple of 256; K = d).  One thread per 16-byte chunk of the output.
__global__ __launch_bounds__(256) void embed_tile_kernel(const bf16_t* __restrict__ E, int V,
                                                         int d, bf16_t* __restrict__ out,
                                                         long chunks) {
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    if (q >= chunks) return;
    const long o = q * 8;                       // output element
    const int c = (int)(o & 31);
    const long i = (o >> 5) & 255;
    const long blk = o >> 13;                   // (row tile, k stage)
    const long ks = blk % (d / 32), rt = blk / (d / 32);
    const long r = rt * 256 + i;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < V) v = *reinterpret_cast<const uint4*>(E + r * d + ks * 32 + c);
    *reinterpret_cast<uint4*>(out + o) = v;
}

// E^T in the blocked layout (rows d, a multiple of 256; K = V): one
// workgroup per 16 KiB output block, 32 rows of E through LDS.
__global__ __launch_bounds__(256) void embed_t_tile_kernel(const bf16_t* __restrict__ E, int V,
                                                           int d, bf16_t* __restrict__ out) {
    __shared__ bf16_t t[32][256 + 8];
    const int vs = blockIdx.x, dt = blockIdx.y;         // v stage (32 entries), d tile (256)
    for (int x = threadIdx.x; x < 32 * 32; x += 256) {  // 32 rows x 32 chunks of 8
        const int j = x / 32, c = (x % 32) * 8;
        const long v = (long)vs * 32 + j;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (v < V) val = *reinterpret_cast<const uint4*>(E + v * d + (long)dt * 256 + c);
        const bf16_t* p = reinterpret_cast<const bf16_t*>(&val);
#pragma unroll
        for (int e = 0; e < 8; ++e) t[j][c + e] = p[e];
    }
    __syncthreads();
    const int i = threadIdx.x;                          // row dt*256 + i of E^T
    bf16_t row[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) row[j] = t[j][i];
    bf16_t* o = out + tiled_index((long)dt * 256 + i, (long)vs * 32, V);
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(o + 8 * q) = *reinterpret_cast<const uint4*>(row + 8 * q);
}

// 64x64 tiles through LDS.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in,
                                                        T* __restrict__ out, int rows,
                                                        int cols) {
    __shared__ T tile[64][65];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        int r = i / 64, c = i % 64;
        if (r0 + r < rows && c0 + c < cols) tile[r][c] = in[(long)(r0 + r) * cols + c0 + c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        int c = i / 64, r = i % 64;
        if (r0 + r < rows && c0 + c < cols) out[(long)(c0 + c) * rows + r0 + r] = tile[r][c];
    }
}

// RoPE of q and k and the K/V cache write; angles in double.
template <typename T>
__global__ __launch_bounds__(256) void rope_kv_kernel(const float* __restrict__ qkv,
                                                      T* __restrict__ q_out, T* __restrict__ kc,
                                                      T* __restrict__ vc, int n, int pos0,
                                                      int cap, int Hq, int Hkv, int dh,
                                                      int rope_on, double log_theta,
                                                      long total) {
    // one thread per (token, head, rotation pair): heads [0, Hq) are query
    // heads, [Hq, Hq + Hkv) key heads (whose value row is copied alongside)
    long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int half = dh / 2;
    const int j = (int)(idx % half);
    const long r = idx / half;
    const int hh = (int)(r % (Hq + Hkv));
    const long t = r / (Hq + Hkv);      // token index b*n + i
    const int b = (int)(t / n), i = (int)(t % n);
    const long pos = pos0 + i;
    float c, s;
    rope_cs(pos, j, dh, rope_on, log_theta, c, s);
    const int width = (Hq + 2 * Hkv) * dh;
    const float* row = qkv + t * width;
    if (hh < Hq) {
        const float x1 = row[hh * dh + j], x2 = row[hh * dh + j + half];
        T* o = q_out + t * (long)Hq * dh + (long)hh * dh;
        o[j] = Elt<T>::from_f(rope_first(x1, x2, c, s));
        o[j + half] = Elt<T>::from_f(rope_second(x1, x2, c, s));
    } else {
        const int h = hh - Hq;
        const float* kr = row + (Hq + h) * dh;
        const float* vr = row + (Hq + Hkv + h) * dh;
        const long slot = (((long)b * Hkv + h) * cap + pos) * dh;
        const float x1 = kr[j], x2 = kr[j + half];
        kc[slot + j] = Elt<T>::from_f(rope_first(x1, x2, c, s));
        kc[slot + j + half] = Elt<T>::from_f(rope_second(x1, x2, c, s));
        vc[slot + j] = Elt<T>::from_f(vr[j]);
        vc[slot + j + half] = Elt<T>::from_f(vr[j + half]);
    }
}

// The same with the stacked Q/K/V product still in split-K partials
// part [splits][rows][width]: each value is first summed over the splits
// exactly as the generic split-K epilogue sums it, so the result equals
// that epilogue followed by rope_kv_kernel, without the fp32 round trip
// and the extra launch.
template <typename T>
__global__ __launch_bounds__(256) void splitk_rope_kv_kernel(const float* __restrict__ part,
                                                             int splits, long rows,
                                                             T* __restrict__ q_out,
                                                             T* __restrict__ kc,
                                                             T* __restrict__ vc, int n, int pos0,
                                                             int cap, int Hq, int Hkv, int dh,
                                                             int rope_on, double log_theta,
                                                             long total) {
    long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int half = dh / 2;
    const int j = (int)(idx % half);
    const long r = idx / half;
    const int hh = (int)(r % (Hq + Hkv));
    const long t = r / (Hq + Hkv);
    const int b = (int)(t / n), i = (int)(t % n);
    const long pos = pos0 + i;
    float c, s;
    rope_cs(pos, j, dh, rope_on, log_theta, c, s);
    const int width = (Hq + 2 * Hkv) * dh;
    const long zs = rows * width;
    const float* row = part + t * width;
    if (hh < Hq) {
        const float x1 = splitk_sum(row + hh * dh + j, zs, splits);
        const float x2 = splitk_sum(row + hh * dh + j + half, zs, splits);
        T* o = q_out + t * (long)Hq * dh + (long)hh * dh;
        o[j] = Elt<T>::from_f(rope_first(x1, x2, c, s));
        o[j + half] = Elt<T>::from_f(rope_second(x1, x2, c, s));
    } else {
        const int h = hh - Hq;
        const float* kr = row + (Hq + h) * dh;
        const float* vr = row + (Hq + Hkv + h) * dh;
        const long slot = (((long)b * Hkv + h) * cap + pos) * dh;
        const float x1 = splitk_sum(kr + j, zs, splits);
        const float x2 = splitk_sum(kr + j + half, zs, splits);
        const float v1 = splitk_sum(vr + j, zs, splits);
        const float v2 = splitk_sum(vr + j + half, zs, splits);
        kc[slot + j] = Elt<T>::from_f(rope_first(x1, x2, c, s));
        kc[slot + j + half] = Elt<T>::from_f(rope_second(x1, x2, c, s));
        vc[slot + j] = Elt<T>::from_f(v1);
        vc[slot + j + half] = Elt<T>::from_f(v2);
    }
}

}  // namespace

template <typename T>
hipError_t rmsnorm(const float* h, const float* w, T* u, int rows, int d, float eps,
                   hipStream_t st, float* u32, uint8_t* q8, uint8_t* q8s) {
    if (rows <= 0) return hipSuccess;
    if (q8 && (d % 32 || !q8s)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_kernel<T>, dim3(rows), dim3(256), 0, st, h, w, u, d, eps, u32, q8,
                       q8s);
    return hipGetLastError();
}

template <typename T>
hipError_t embed_rows(const T* E, int V, const int32_t* tok, int ld, int n, int B, float* h, int d,
                      hipStream_t st) {
    if (n <= 0 || B <= 0) return hipSuccess;
    hipLaunchKernelGGL(embed_kernel<T>, dim3(B * n), dim3(256), 0, st, E, tok, ld, n, V, h, d);
    return hipGetLastError();
}

template <typename T>
hipError_t splitk_reduce(const float* part, T* out, int splits, int rows, int cols,
                         hipStream_t st, const float* row_stats) {
    long total = (long)rows * cols;
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(splitk_reduce_kernel<T>, dim3((unsigned)cdiv((int)total, 256)), dim3(256),
                       0, st, part, out, splits, total, cols, row_stats);
    return hipGetLastError();
}

template <typename T>
hipError_t selfcond_topk(const T* E, int d, const int32_t* idx, const float* p, int K, int rows,
                         T* out, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (d % 8 || K < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(selfcond_topk_kernel<T>, dim3(rows), dim3(256), 0, st, E, d, idx, p, K, out);
    return hipGetLastError();
}
template hipError_t selfcond_topk<bf16_t>(const bf16_t*, int, const int32_t*, const float*, int, int,
                                          bf16_t*, hipStream_t);
template hipError_t selfcond_topk<float>(const float*, int, const int32_t*, const float*, int, int,
                                         float*, hipStream_t);

hipError_t rmsnorm_tiled(const float* h, const float* w, uint16_t* u, int rows, int d, float eps,
                         hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(rmsnorm_tiled_kernel, dim3(rows), dim3(256), 0, st, h, w, u, d, eps);
    return hipGetLastError();
}

hipError_t embed_tile(const uint16_t* E, int V, int d, int transpose, uint16_t* out,
                      hipStream_t st) {
    if (transpose) {
        if (d % 256 || V % 32) return hipErrorInvalidValue;
        hipLaunchKernelGGL(embed_t_tile_kernel, dim3(V / 32, d / 256), dim3(256), 0, st, E, V, d, out);
    } else {
        if (d % 32) return hipErrorInvalidValue;
        const long chunks = (long)cdiv(V, 256) * 256 * d / 8;
        hipLaunchKernelGGL(embed_tile_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st,
                           E, V, d, out, chunks);
    }
    return hipGetLastError();
}

hipError_t fill_i32(int32_t* p, int32_t v, long n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, v, n);
    return hipGetLastError();
}

hipError_t widen_bf16(const bf16_t* in, float* out, long n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(widen_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, in, out, n);
    return hipGetLastError();
}

template <typename T>
hipError_t transpose(const T* in, T* out, int rows, int cols, hipStream_t st) {
    dim3 grid(cdiv(cols, 64), cdiv(rows, 64));
    hipLaunchKernelGGL(transpose_kernel<T>, grid, dim3(256), 0, st, in, out, rows, cols);
    return hipGetLastError();
}

template <typename T>
hipError_t rope_kv(const float* qkv, T* q_out, T* kc, T* vc, int B, int n, int pos0, int cap,
                   int Hq, int Hkv, int dh, int rope_on, float theta, hipStream_t st) {
    long total = (long)B * n * (Hq + Hkv) * (dh / 2);
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(rope_kv_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, qkv, q_out, kc, vc, n, pos0, cap, Hq, Hkv, dh, rope_on,
                       log((double)theta), total);
    return hipGetLastError();
}

template <typename T>
hipError_t splitk_rope_kv(const float* part, int splits, T* q_out, T* kc, T* vc, int B, int n,
                          int pos0, int cap, int Hq, int Hkv, int dh, int rope_on, float theta,
                          hipStream_t st) {
    long total = (long)B * n * (Hq + Hkv) * (dh / 2);
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(splitk_rope_kv_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, st, part, splits, (long)B * n, q_out, kc, vc, n, pos0, cap, Hq, Hkv, dh,
                       rope_on, log((double)theta), total);
    return hipGetLastError();
}

template <typename T>
hipError_t splitk_add_norm(const float* part, int splits, float* h, int rows, int d,
                           const float* w, T* u, float eps, hipStream_t st, float* u32,
                           uint8_t* q8, uint8_t* q8s) {
    if (rows <= 0) return hipSuccess;
    if (d % 4 || (q8 && (d % 32 || !q8s))) return hipErrorInvalidValue;
    hipLaunchKernelGGL(splitk_add_norm_kernel<T>, dim3(rows), dim3(256), 0, st, part, splits,
                       (long)rows, h, w, u, d, eps, u32, q8, q8s);
    return hipGetLastError();
}

#define DG_INST(T)                                                                        \
    template hipError_t rmsnorm<T>(const float*, const float*, T*, int, int, float,        \
                                   hipStream_t, float*, uint8_t*, uint8_t*);               \
    template hipError_t embed_rows<T>(const T*, int, const int32_t*, int, int, int, float*, int, \
                                      hipStream_t);                                        \
    template hipError_t splitk_reduce<T>(const float*, T*, int, int, int, hipStream_t,     \
                                         const float*);                                    \
    template hipError_t transpose<T>(const T*, T*, int, int, hipStream_t);                 \
    template hipError_t rope_kv<T>(const float*, T*, T*, T*, int, int, int, int, int, int, \
                                   int, int, float, hipStream_t);                          \
    template hipError_t splitk_rope_kv<T>(const float*, int, T*, T*, T*, int, int, int, int, \
                                          int, int, int, int, float, hipStream_t); \
    template hipError_t splitk_add_norm<T>(const float*, int, float*, int, int, const float*, \
                                           T*, float, hipStream_t, float*, uint8_t*, uint8_t*);
DG_INST(bf16_t)
DG_INST(float)
#undef DG_INST

}  // namespace dg
