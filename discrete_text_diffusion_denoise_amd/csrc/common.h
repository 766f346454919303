// Shared device-side helpers for the gfx950 kernels: element types, bf16
// conversion, MFMA fragment types and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 storage
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define DG_WAVE 64

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Round to nearest even (NaN stays NaN): gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Maximum under which a NaN ranks above every number (a NaN operand wins).
// The slab maxima that steer the sampler's top-k candidate search use it, so
// that a NaN or an infinite logit always reaches the candidates and its row's
// statistics turn NaN (the row is then reported as non-finite).
__device__ __forceinline__ float max_nan(float a, float b) { return (a != a || a > b) ? a : b; }

// Element-type traits: loading/storing 8 consecutive k-values of a fragment.
template <typename T> struct Elt;

template <> struct Elt<bf16_t> {
    static constexpr int bytes = 2;
    static __device__ __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
    static __device__ __forceinline__ bf16_t from_f(float v) { return f2bf(v); }
};
template <> struct Elt<float> {
    static constexpr int bytes = 4;
    static __device__ __forceinline__ float to_f(float v) { return v; }
    static __device__ __forceinline__ float from_f(float v) { return v; }
};

// A fragment of 8 k-values per lane.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
    uint4 v;  // 8 bf16
};
template <> struct Frag<float> {
    float4 lo, hi;  // 8 fp32
};

// acc += A_frag * B_frag over 32 k (16x16 output tile).
// Lane l holds A row (l & 15), B column (l & 15); its 8 values are the same
// 8 k-indices in both operands, so any assignment of physical k to
// (lane group, element) gives the same sum.  Output: lane l holds rows
// 4*(l>>4)+i, column l & 15.
__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
    bf16x8_t av = __builtin_bit_cast(bf16x8_t, a.v);
    bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b.v);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<float>& a, const Frag<float>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// Load 8 consecutive elements at p (16-byte aligned for bf16, 32 for f32).
__device__ __forceinline__ void load_frag(Frag<bf16_t>& f, const bf16_t* p) {
    f.v = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
    f.lo = *reinterpret_cast<const float4*>(p);
    f.hi = *reinterpret_cast<const float4*>(p + 4);
}
__device__ __forceinline__ void zero_frag(Frag<bf16_t>& f) { f.v = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero_frag(Frag<float>& f) {
    f.lo = make_float4(0.f, 0.f, 0.f, 0.f);
    f.hi = f.lo;
}

// Convert 8 floats to a fragment of T.
__device__ __forceinline__ void frag_from_f(Frag<bf16_t>& f, const float* x) {
    f.v.x = pack_bf2(x[0], x[1]);
    f.v.y = pack_bf2(x[2], x[3]);
    f.v.z = pack_bf2(x[4], x[5]);
    f.v.w = pack_bf2(x[6], x[7]);
}
__device__ __forceinline__ void frag_from_f(Frag<float>& f, const float* x) {
    f.lo = make_float4(x[0], x[1], x[2], x[3]);
    f.hi = make_float4(x[4], x[5], x[6], x[7]);
}

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Sum of a split-K product's partials for one output, in split order:
// pp points at the element in split 0, splits are zs floats apart; up to
// eight loads go out before their adds (a short last group is predicated,
// not a loop of dependent loads).  Every epilogue that reduces partials uses
// it, so they give the same bits.
__device__ __forceinline__ float splitk_sum(const float* pp, long zs, int splits) {
    float v = 0.f;
    for (int z = 0; z < splits; z += 8) {
        float p[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) p[q] = z + q < splits ? pp[(z + q) * zs] : 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (z + q < splits) v += p[q];
    }
    return v;
}

// splitk_sum of four adjacent outputs (pp 16-byte aligned, zs a multiple of
// 4): each component summed in the same order as splitk_sum sums it
__device__ __forceinline__ float4 splitk_sum4(const float* pp, long zs, int splits) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z = 0; z < splits; z += 8) {
        float4 p[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            p[q] = z + q < splits ? *reinterpret_cast<const float4*>(pp + (z + q) * zs)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (z + q < splits) {
                v.x += p[q].x;
                v.y += p[q].y;
                v.z += p[q].z;
                v.w += p[q].w;
            }
    }
    return v;
}

// RMSNorm arithmetic shared by every kernel that normalises rows of d fp32
// values with 256 threads (thread t takes the float4 at 4t + 1024 i), so that
// they give the same bits: the sum of squares in fixed fma order, the block
// total over the four waves in wave order, the scale and the scaled value.
__device__ __forceinline__ float rms_accum(float ss, float4 v) {
    ss = __builtin_fmaf(v.x, v.x, ss);
    ss = __builtin_fmaf(v.y, v.y, ss);
    ss = __builtin_fmaf(v.z, v.z, ss);
    return __builtin_fmaf(v.w, v.w, ss);
}
// the row's scale 1 / sqrt(mean square + eps); part: 4 floats of LDS
__device__ __forceinline__ float rms_block_scale(float ss, float* part, int d, float eps) {
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = part[0] + part[1] + part[2] + part[3];
    return 1.0f / sqrtf(tot / (float)d + eps);
}
__device__ __forceinline__ float4 rms_apply(float4 v, float scale, const float* w, int i) {
    const float4 s = w ? *reinterpret_cast<const float4*>(w + i) : make_float4(1.f, 1.f, 1.f, 1.f);
    return make_float4(v.x * scale * s.x, v.y * scale * s.y, v.z * scale * s.z, v.w * scale * s.w);
}

// RoPE rotation of pair j (of dh / 2) at position pos: angle pos * theta^(-2j/dh)
// in double, cos and sin rounded to float, then (x1, x2) -> (x1 c - x2 s, x2 c + x1 s)
__device__ __forceinline__ void rope_cs(long pos, int j, int dh, int rope_on, double log_theta,
                                        float& c, float& s) {
    c = 1.f;
    s = 0.f;
    if (rope_on) {
        const double inv_freq = exp(-2.0 * (double)j / (double)dh * log_theta);
        const double ang = (double)pos * inv_freq;
        c = (float)cos(ang);
        s = (float)sin(ang);
    }
}
__device__ __forceinline__ float rope_first(float x1, float x2, float c, float s) {
    return x1 * c - x2 * s;
}
__device__ __forceinline__ float rope_second(float x1, float x2, float c, float s) {
    return x2 * c + x1 * s;
}
