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
