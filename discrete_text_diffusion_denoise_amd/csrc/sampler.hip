// Multinomial-diffusion sampler on gfx950.
//
// Report-summary page (animattoys.com), section 1: uncertain positions are
// replaced by any vocabulary token, and locked tokens can still change in a
// later round; section 4: order positions by entropy and lock from the most
// certain while the running entropy stays within the budget, re-randomise the
// rest, temperature falls linearly, stop once the mean entropy is small and
// the most likely sequence is unchanged, within a round budget.
//
// The arithmetic is fixed exactly (the pages leave it open) so that decisions
// are bit-reproducible:
//   E(x)  e^x for x <= 0: Cody-Waite reduction with a two-part ln2, Taylor
//         polynomial of degree 6 in Horner form with fma, 2^k from exponent
//         bits; x < -87 gives 0 (never subnormal).
//   L(x)  ln x for x >= 1: mantissa in (sqrt(1/2), sqrt(2)], 2*atanh series
//         to f^13 with fma, two-part ln2.
//   Row layout: 65536-entry tiles; chunk c = t*1024 + lam holds entries
//         4*(t*16384 + d*1024 + lam) + q, d < 16, q < 4, in increasing order.
//   Chunk record: max, first argmax, sequential sums of E(z), E(z)*z and
//         E(z/T) with z = l - max.  Records merge by a symmetric rule; the row
//         record folds each lane's tiles in order and then reduces over the
//         1024 lanes by a pairwise tree (adjacent pairs first).
//   Draw: three inverse-CDF picks (64-chunk superchunks, chunks, entries),
//         each "first running sum > u * total, else last positive", with
//         u = (2r+1)/2^24 from Philox4x64-10 words 0, 2 and 3; word 1 gives
//         the renoise token mulhi(word, V).
// Every float operation below is one IEEE binary32 operation in the order
// written; contraction into fma is disabled for this file.
#pragma clang fp contract(off)

#include "common.h"
#include "kernels.h"

namespace dg {

namespace {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int NLANE = 1024;
constexpr int NDEPTH = 16;
constexpr int TILE = 4 * NLANE * NDEPTH;
constexpr int SUPER = 64;

// Computed for every x and selected at the end (no branch): the value for
// x >= -87 is the same sequence of operations either way.
__device__ __forceinline__ float dexp(float x) {
    const float LOG2E = 1.44269504088896341f;
    const float LN2_HI = 0.693145751953125f;
    const float LN2_LO = 1.42860682030941723e-06f;
    float kf = __builtin_rintf(x * LOG2E);
    float r = __builtin_fmaf(-kf, LN2_HI, x);
    r = __builtin_fmaf(-kf, LN2_LO, r);
    float p = 1.0f / 720.0f;
    p = __builtin_fmaf(p, r, 1.0f / 120.0f);
    p = __builtin_fmaf(p, r, 1.0f / 24.0f);
    p = __builtin_fmaf(p, r, 1.0f / 6.0f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    // p * 2^k: for x >= -87, k >= -126 and p > 1, so the product is a normal
    // number and scaling the exponent (ldexp) is the same exact result
    const float v = __builtin_amdgcn_ldexpf(p, (int)kf);
    return x >= -87.0f ? v : 0.0f;
}

// Self-conditioning weight of an entry: e = E(l - m_c) against its chunk's
// max, f = E(m_c - M) the chunk's factor against the row max; e * f is
// exp(l - M) to within a few binary32 roundings.  The sampler's row pass and
// the stand-alone probability pass both compute it this way, chunk by chunk,
// so their outputs are the same bits.
__device__ __forceinline__ float chunk_weight(float e, float f) { return e * f; }

__device__ __forceinline__ float dlog(float x) {
    const float LN2_HI = 0.693145751953125f;
    const float LN2_LO = 1.42860682030941723e-06f;
    const uint32_t b = __float_as_uint(x);
    int e = (int)((b >> 23) & 0xffu) - 127;
    float m = __uint_as_float((b & 0x7fffffu) | 0x3f800000u);
    if (m > 1.41421356f) {
        m = m * 0.5f;
        e = e + 1;
    }
    const float f = (m - 1.0f) / (m + 1.0f);
    const float f2 = f * f;
    float q = 1.0f / 13.0f;
    q = __builtin_fmaf(q, f2, 1.0f / 11.0f);
    q = __builtin_fmaf(q, f2, 1.0f / 9.0f);
    q = __builtin_fmaf(q, f2, 1.0f / 7.0f);
    q = __builtin_fmaf(q, f2, 1.0f / 5.0f);
    q = __builtin_fmaf(q, f2, 1.0f / 3.0f);
    q = __builtin_fmaf(q, f2, 1.0f);
    const float lm = (2.0f * f) * q;
    const float ef = (float)e;
    return __builtin_fmaf(ef, LN2_HI, __builtin_fmaf(ef, LN2_LO, lm));
}

// Philox4x64-10 (Salmon et al., SC'11).
__device__ __forceinline__ void philox(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                       uint64_t k0, uint64_t k1, uint64_t o[4]) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
        const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    o[0] = c0;
    o[1] = c1;
    o[2] = c2;
    o[3] = c3;
}

__device__ __forceinline__ float uniform01(uint64_t w) {
    const uint32_t r = (uint32_t)(w >> 41);
    return (float)(2u * r + 1u) * 5.9604644775390625e-08f;
}
__device__ __forceinline__ int32_t uniform_token(uint64_t w, int V) {
    return (int32_t)__umul64hi(w, (uint64_t)(uint32_t)V);
}

struct Rec {
    float m;
    int j;
    float s, a;
};

__device__ __forceinline__ Rec merge(const Rec& x, const Rec& y) {
    if (x.s == 0.0f) return y;
    if (y.s == 0.0f) return x;
    Rec r;
    r.m = x.m > y.m ? x.m : y.m;
    r.j = x.m > y.m ? x.j : (y.m > x.m ? y.j : (x.j < y.j ? x.j : y.j));
    const float dx = x.m - r.m, dy = y.m - r.m;
    const float fx = dexp(dx), fy = dexp(dy);
    const float sx = x.s * fx, sy = y.s * fy;
    r.s = sx + sy;
    const float ax = fx * (x.a + dx * x.s);
    const float ay = fy * (y.a + dy * y.s);
    r.a = ax + ay;
    return r;
}

__device__ __forceinline__ Rec shfl_rec(const Rec& x, int mask) {
    Rec o;
    o.m = __shfl_xor(x.m, mask, 64);
    o.j = __shfl_xor(x.j, mask, 64);
    o.s = __shfl_xor(x.s, mask, 64);
    o.a = __shfl_xor(x.a, mask, 64);
    return o;
}

// First index whose running sum exceeds u * total, else the last positive.
__device__ int pick_seq(const float* w, int n, float u) {
    float total = 0.0f;
    for (int i = 0; i < n; ++i) total = total + w[i];
    const float target = u * total;
    float acc = 0.0f;
    for (int i = 0; i < n; ++i) {
        acc = acc + w[i];
        if (acc > target) return i;
    }
    for (int i = n - 1; i >= 0; --i)
        if (w[i] > 0.0f) return i;
    return 0;
}

// pick_seq over an array in LDS, read 16 values at a time (4 x 16 bytes,
// one wait) instead of one wait per value: the same sums in the same order.
// w is 16-byte aligned and readable up to n rounded up to 16.
__device__ int pick_lds(const float* w, int n, float u) {
    float total = 0.0f;
    for (int i0 = 0; i0 < n; i0 += 16) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 t = reinterpret_cast<const float4*>(w + i0)[q];
            v[4 * q + 0] = t.x;
            v[4 * q + 1] = t.y;
            v[4 * q + 2] = t.z;
            v[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (i0 + j < n) total = total + v[j];
    }
    const float target = u * total;
    float acc = 0.0f;
    for (int i0 = 0; i0 < n; i0 += 16) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 t = reinterpret_cast<const float4*>(w + i0)[q];
            v[4 * q + 0] = t.x;
            v[4 * q + 1] = t.y;
            v[4 * q + 2] = t.z;
            v[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (i0 + j < n) {
                acc = acc + v[j];
                if (acc > target) return i0 + j;
            }
        }
    }
    for (int i = n - 1; i >= 0; --i)
        if (w[i] > 0.0f) return i;
    return 0;
}

// Raw buffer resource over `bytes` bytes at p (gfx9 word 3: 32-bit data,
// no swizzle).  A buffer access takes one 32-bit lane offset plus a uniform
// offset, so the sixteen loads and stores of a tile share one address
// register instead of a 64-bit address each.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Where a row's self-conditioning weights go: a buffer over the row's span
// of the output, 64-wide blocked (entry k at (k / 64) * 16384 + k % 64
// elements from the row's first one, tiled64_index) or row-major, and the
// row max M.
struct ProbOut {
    __amdgpu_buffer_rsrc_t rs;
    int tiled;
    float M;
    __device__ uint32_t off(uint32_t k) const {   // byte offset of entry k
        return tiled ? 2u * (((k >> 6) << 14) + (k & 63)) : 2u * k;
    }
    __device__ int step() const { return tiled ? (2 << 20) : 8192; }   // entries k -> k + 4096
};

// Weights of four consecutive entries k..k+3 (k % 4 == 0): lane part and
// uniform part of the byte offset.  Non-temporal (the operand is read once,
// by the next round's product): measured faster for whole 128-byte lines.
__device__ __forceinline__ void put4(const ProbOut& po, uint32_t voff, int soff, const float (&w)[4]) {
    __builtin_amdgcn_raw_buffer_store_b64(
        __builtin_bit_cast(u32x2_t, make_uint2(pack_bf2(w[0], w[1]), pack_bf2(w[2], w[3]))), po.rs,
        voff, soff, 2 /* nt */);
}

// Record of a whole chunk (all 64 entries members; x in member order, k0 its
// first entry); *s2 receives its weight sum at temperature T.  With PROBS,
// also the self-conditioning weights of its entries.
template <bool PROBS>
__device__ __forceinline__ Rec chunk_full(const float (&x)[4 * NDEPTH], int k0, float invT,
                                          float* s2out, const ProbOut& po) {
    // chunk max (each entry replaces it only if strictly greater, in member
    // order), then the first member equal to it: the same first argmax as
    // tracking both in one pass, since the max is attained first there (+0
    // and -0 compare equal in both passes; NaN is never taken, and a NaN
    // first entry leaves the max NaN and the argmax 0)
    float m = x[0];
#pragma unroll
    for (int u = 1; u < 4 * NDEPTH; ++u) m = x[u] > m ? x[u] : m;
    int ju = 0;
#pragma unroll
    for (int u = 4 * NDEPTH - 1; u > 0; --u) ju = x[u] == m ? u : ju;
    // byte offset of entry k0 in the output; entry k0 + 4096 d adds step d
    const uint32_t o0 = PROBS ? po.off((uint32_t)k0) : 0u;
    const int ds = PROBS ? po.step() : 0;
    const float f = PROBS ? dexp(m - po.M) : 0.0f;
    float w[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float sum = 0.0f, ac = 0.0f, s2 = 0.0f;
    if (invT != 1.0f) {
#pragma unroll
        for (int u = 0; u < 4 * NDEPTH; ++u) {
            const float z = x[u] - m;
            const float e = dexp(z);
            sum = sum + e;
            const float ez = e * z;
            ac = ac + ez;
            s2 = s2 + dexp(z * invT);
            if (PROBS) {
                w[u % 4] = chunk_weight(e, f);
                if (u % 4 == 3) put4(po, o0, ds * (u / 4), w);
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < 4 * NDEPTH; ++u) {
            const float z = x[u] - m;
            const float e = dexp(z);
            sum = sum + e;
            const float ez = e * z;
            ac = ac + ez;
            if (PROBS) {
                w[u % 4] = chunk_weight(e, f);
                if (u % 4 == 3) put4(po, o0, ds * (u / 4), w);
            }
        }
        s2 = sum;
    }
    *s2out = s2;
    Rec r;
    r.m = m;
    r.j = k0 + 4 * NLANE * (ju / 4) + (ju % 4);
    // a chunk whose maximum is not finite is marked by a NaN sum, so that
    // every non-finite logit makes its row's entropy NaN
    r.s = (m - m == 0.0f) ? sum : __builtin_nanf("");
    r.a = ac;
    return r;
}

// Chunk lam of the ragged last tile t: members are the entries below V.
template <bool VEC, bool PROBS>
__device__ __forceinline__ Rec chunk_ragged(const float* row, int V, int t, int lam, float invT,
                                            float* s2out, const ProbOut& po) {
    float x[4 * NDEPTH];
    Rec rc = {-INFINITY, -1, 0.0f, 0.0f};
    float s2 = 0.0f;
    const long g0 = (long)t * (NLANE * NDEPTH) + lam;
#pragma unroll
    for (int d = 0; d < NDEPTH; ++d) {
        const long k = 4 * (g0 + (long)d * NLANE);
        if (VEC && k + 3 < V) {
            const float4 v = *reinterpret_cast<const float4*>(row + k);
            x[4 * d + 0] = v.x;
            x[4 * d + 1] = v.y;
            x[4 * d + 2] = v.z;
            x[4 * d + 3] = v.w;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) x[4 * d + q] = (k + q < V) ? row[k + q] : -INFINITY;
        }
    }
    float m = -INFINITY;
    int j = -1;
#pragma unroll
    for (int d = 0; d < NDEPTH; ++d)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const long k = 4 * (g0 + (long)d * NLANE) + q;
            if (k < V && (x[4 * d + q] > m || j < 0)) {
                m = x[4 * d + q];
                j = (int)k;
            }
        }
    if (j >= 0) {
        const float f = PROBS ? dexp(m - po.M) : 0.0f;
        float sum = 0.0f, ac = 0.0f;
#pragma unroll
        for (int d = 0; d < NDEPTH; ++d) {
            float w[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const long k = 4 * (g0 + (long)d * NLANE) + q;
                if (k < V) {
                    const float z = x[4 * d + q] - m;
                    const float e = dexp(z);
                    sum = sum + e;
                    const float ez = e * z;
                    ac = ac + ez;
                    if (invT != 1.0f) s2 = s2 + dexp(z * invT);
                    if (PROBS) w[q] = chunk_weight(e, f);
                }
            }
            const uint32_t k = 4u * (uint32_t)(g0 + (long)d * NLANE);
            if (PROBS && k + 3 < (uint32_t)V) put4(po, po.off(k), 0, w);
        }
        if (invT == 1.0f) s2 = sum;
        rc.m = m;
        rc.j = j;
        rc.s = (m - m == 0.0f) ? sum : __builtin_nanf("");
        rc.a = ac;
    }
    *s2out = s2;
    return rc;
}

// One workgroup of 512 threads per logit row; thread p owns chunks p and
// p + 512 of every tile (256 registers a lane at this size, where 1024
// threads of 128 spill).
constexpr int NTHR = 512;

template <bool VEC, bool PROBS>
__global__ __launch_bounds__(NTHR) void sample_row_kernel(SampleArgs a) {
    extern __shared__ __align__(16) float sm[];
    const int nt = cdiv(a.V, TILE);
    float* Gs = sm;                       // [nt*1024] chunk weights at temperature T
    float* Ms = sm + nt * NLANE;          // [nt*1024] chunk maxima
    __shared__ Rec wrec[16];
    __shared__ __align__(16) float Wsup[8 * 16];
    __shared__ __align__(16) float wk[4 * NDEPTH];
    __shared__ int kk[4 * NDEPTH];
    __shared__ int nmem;

    const long rowid = blockIdx.x;        // b*N + i
    const int b = (int)(rowid / a.N), i = (int)(rowid % a.N);
    if (a.stop && a.stop[b]) return;
    const float* row = a.logits + rowid * (long)a.V;
    const __amdgpu_buffer_rsrc_t lrs = buf_rsrc(row, 4u * (uint32_t)a.V);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float invT = a.inv_t;

    // Optional output for the next round's self-conditioning: the weight
    // chunk_weight(E(l - m_c), E(m_c - M)) of every logit, m_c its chunk's
    // max and M the row max (the largest of the head GEMM's slab maxima), as
    // bf16, blocked or row-major.  E(l - m_c) is the value the statistics
    // below sum anyway.  It takes no part in the decisions.
    __shared__ float wmx[NTHR / 64];
    ProbOut po;
    po.rs = buf_rsrc(a.probs, 0);   // an empty resource when unused
    po.tiled = a.probs_tiled;
    po.M = 0.0f;
    if (PROBS) {
        const float* rm = a.rowmax + rowid * (long)a.rowmax_n;
        float mm = -INFINITY;
        for (int c = tid; c < a.rowmax_n; c += NTHR) mm = fmaxf(mm, rm[c]);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) mm = fmaxf(mm, __shfl_xor(mm, o, 64));
        if (lane == 0) wmx[wave] = mm;
        __syncthreads();
        float Mp = wmx[0];
#pragma unroll
        for (int w = 1; w < NTHR / 64; ++w) Mp = fmaxf(Mp, wmx[w]);
        po.M = Mp;
        // the row's span fits 32 bits (V <= 2^19)
        if (po.tiled)
            po.rs = buf_rsrc(a.probs + tiled64_index(rowid, 0, a.V),
                             2u * ((((uint32_t)a.V / 64 - 1) << 14) + 64));
        else
            po.rs = buf_rsrc(a.probs + rowid * (long)a.V, 2u * (uint32_t)a.V);
    }

    // lane records of chunks tid (F0) and tid + 512 (F1), folded over the
    // tiles in order: whole tiles first (every entry a member), then the
    // ragged last tile
    Rec F0 = {-INFINITY, -1, 0.0f, 0.0f}, F1 = F0;
    const int nfull = VEC ? a.V / TILE : 0;
    for (int t = 0; t < nfull; ++t) {
        float x0[4 * NDEPTH], x1[4 * NDEPTH];
        const int k0 = 4 * (t * (NLANE * NDEPTH) + tid), k1 = k0 + 4 * NTHR;
        // entry k0 + 4096 d is 16 KiB d after entry k0
#pragma unroll
        for (int d = 0; d < NDEPTH; ++d) {
            const f32x4_t v = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(lrs, 4u * (uint32_t)k0, 16384 * d, 0));
            x0[4 * d + 0] = v[0];
            x0[4 * d + 1] = v[1];
            x0[4 * d + 2] = v[2];
            x0[4 * d + 3] = v[3];
        }
        float s0, s1;
        const Rec r0 = chunk_full<PROBS>(x0, k0, invT, &s0, po);
        // the second chunk's loads go out after the first chunk's work
        // (measured: fewer loads in flight beside the first chunk's stores,
        // and the other wave of the SIMD covers their latency)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < NDEPTH; ++d) {
            const f32x4_t v = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(lrs, 4u * (uint32_t)k1, 16384 * d, 0));
            x1[4 * d + 0] = v[0];
            x1[4 * d + 1] = v[1];
            x1[4 * d + 2] = v[2];
            x1[4 * d + 3] = v[3];
        }
        const Rec r1 = chunk_full<PROBS>(x1, k1, invT, &s1, po);
        Gs[t * NLANE + tid] = s0;
        Ms[t * NLANE + tid] = r0.m;
        Gs[t * NLANE + tid + NTHR] = s1;
        Ms[t * NLANE + tid + NTHR] = r1.m;
        F0 = (t == 0) ? r0 : merge(F0, r0);
        F1 = (t == 0) ? r1 : merge(F1, r1);
    }
    for (int t = nfull; t < nt; ++t) {
        float s0, s1;
        const Rec r0 = chunk_ragged<VEC, PROBS>(row, a.V, t, tid, invT, &s0, po);
        const Rec r1 = chunk_ragged<VEC, PROBS>(row, a.V, t, tid + NTHR, invT, &s1, po);
        Gs[t * NLANE + tid] = s0;
        Ms[t * NLANE + tid] = r0.m;
        Gs[t * NLANE + tid + NTHR] = s1;
        Ms[t * NLANE + tid + NTHR] = r1.m;
        F0 = (t == 0) ? r0 : merge(F0, r0);
        F1 = (t == 0) ? r1 : merge(F1, r1);
    }
    // pairwise tree over the 1024 chunk lanes: within each group of 64
    // (F0 of wave w is group w, F1 group w + 8), then over the 16 groups.
    // merge is symmetric, so the butterfly leaves every lane of a pair with
    // the record of the pair: level by level the same tree as merging
    // adjacent pairs first.
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        F0 = merge(F0, shfl_rec(F0, o));
        F1 = merge(F1, shfl_rec(F1, o));
    }
    if (lane == 0) {
        wrec[wave] = F0;
        wrec[wave + NTHR / 64] = F1;
    }
    __syncthreads();
    __shared__ Rec rowrec;
    if (wave == 0) {
        Rec W = wrec[lane & 15];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) W = merge(W, shfl_rec(W, o));
        if (lane == 0) rowrec = W;
    }
    __syncthreads();
    const Rec R = rowrec;

    if (a.stats_only) {
        if (tid == 0) {
            if (a.stats) {
                float H = dlog(R.s) - R.a / R.s;
                H = H > 0.0f ? H : (H != H ? H : 0.0f);  // NaN (non-finite logits) stays NaN
                float* st = a.stats + rowid * 4;
                st[0] = R.m;
                st[1] = R.s;
                st[2] = H;
                st[3] = 1.0f / R.s;
            }
            if (a.newmax) a.newmax[rowid] = R.j;
            if (a.loss) {
                const int x = a.target[rowid];
                a.loss[rowid] = (x >= 0 && x < a.V) ? dlog(R.s) - (row[x] - R.m) : NAN;
            }
        }
        return;
    }

    // chunk weights at temperature T, relative to the row max
    for (int c = tid; c < nt * NLANE; c += NTHR) {
        const float s2 = Gs[c];
        Gs[c] = s2 == 0.0f ? 0.0f : s2 * dexp((Ms[c] - R.m) * invT);
    }
    __syncthreads();
    const int nsup = nt * (NLANE / SUPER);
    if (tid < nsup) {
        // sequential sum of the superchunk's 64 chunk weights, read 16 at a time
        const float4* g4p = reinterpret_cast<const float4*>(Gs + tid * SUPER);
        float acc = 0.0f;
        for (int l0 = 0; l0 < SUPER / 4; l0 += 4) {
            float4 t[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) t[q] = g4p[l0 + q];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = acc + t[q].x;
                acc = acc + t[q].y;
                acc = acc + t[q].z;
                acc = acc + t[q].w;
            }
        }
        Wsup[tid] = acc;
    }
    __syncthreads();
    __shared__ int cstar_s;
    __shared__ uint64_t words[4];
    if (tid == 0) {
        uint64_t o[4];
        philox((uint64_t)a.step, (uint64_t)b, (uint64_t)i, 0ull, a.seed, 0ull, o);
        words[0] = o[0];
        words[1] = o[1];
        words[2] = o[2];
        words[3] = o[3];
        const int sstar = pick_lds(Wsup, nsup, uniform01(o[0]));
        cstar_s = sstar * SUPER + pick_lds(Gs + sstar * SUPER, SUPER, uniform01(o[2]));
    }
    __syncthreads();
    // entries of the chosen chunk, in member order
    const int cstar = cstar_s;
    if (tid < 4 * NDEPTH) {
        const int t = cstar / NLANE, l = cstar % NLANE;
        const int d = tid / 4, q = tid % 4;
        const long k = 4 * ((long)t * NLANE * NDEPTH + (long)d * NLANE + l) + q;
        wk[tid] = k < a.V ? dexp((row[k] - Ms[cstar]) * invT) : 0.0f;
        kk[tid] = k < a.V ? (int)k : -1;
        // k grows with tid, so the members (k < V) are the first popcount
        // slots, already in member order
        const uint64_t mem = __ballot(k < a.V);
        if (tid == 0) nmem = __popcll(mem);
    }
    __syncthreads();
    if (tid == 0) {
        const int n = nmem;
        const int yv = n > 0 ? kk[pick_lds(wk, n, uniform01(words[3]))] : 0;
        float H = dlog(R.s) - R.a / R.s;
        H = H > 0.0f ? H : (H != H ? H : 0.0f);  // NaN (non-finite logits) stays NaN
        const float pmax = 1.0f / R.s;
        float* st = a.stats + rowid * 4;
        st[0] = R.m;
        st[1] = R.s;
        st[2] = H;
        st[3] = pmax;
        a.newmax[rowid] = R.j;
        a.y[rowid] = yv;
        a.r[rowid] = uniform_token(words[1], a.V);
    }
}

// Stand-alone pass: the self-conditioning weights of whole rows from their
// statistics (M = stats[0], the row max the statistics hold), chunk by chunk
// exactly as the row pass computes them.  blockIdx.x = row, blockIdx.y = a
// quarter of one tile's 1024 chunks.  V % 4 == 0.
__global__ __launch_bounds__(256) void selfcond_probs_kernel(const float* __restrict__ logits,
                                                            const float* __restrict__ stats,
                                                            bf16_t* __restrict__ out, int V,
                                                            const int32_t* halt, int tiled) {
    if (halt && *halt) return;
    const long rowid = blockIdx.x;
    const int t = blockIdx.y >> 2;
    const int lam = ((blockIdx.y & 3) << 8) + threadIdx.x;
    const float M = stats[rowid * 4];
    const float* row = logits + rowid * (long)V;
    const long g0 = (long)t * (NLANE * NDEPTH) + lam;
    float x[4 * NDEPTH];
#pragma unroll
    for (int d = 0; d < NDEPTH; ++d) {
        const long k = 4 * (g0 + (long)d * NLANE);
        const float4 v = k + 3 < V ? *reinterpret_cast<const float4*>(row + k)
                                   : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        x[4 * d + 0] = v.x;
        x[4 * d + 1] = v.y;
        x[4 * d + 2] = v.z;
        x[4 * d + 3] = v.w;
    }
    // the chunk max as the row pass takes it: the first member, then every
    // member that is strictly greater, in member order
    float m = -INFINITY;
    bool any = false;
#pragma unroll
    for (int u = 0; u < 4 * NDEPTH; ++u) {
        const long k = 4 * (g0 + (long)(u / 4) * NLANE) + u % 4;
        if (k < V && (!any || x[u] > m)) {
            m = x[u];
            any = true;
        }
    }
    if (!any) return;
    const float f = dexp(m - M);
#pragma unroll
    for (int d = 0; d < NDEPTH; ++d) {
        const long k = 4 * (g0 + (long)d * NLANE);
        if (k + 3 < V) {
            float w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = chunk_weight(dexp(x[4 * d + q] - m), f);
            const long o = tiled ? tiled64_index(rowid, k, V) : rowid * (long)V + k;
            *reinterpret_cast<uint2*>(out + o) = make_uint2(pack_bf2(w[0], w[1]), pack_bf2(w[2], w[3]));
        }
    }
}

// ---------------------------------------------------------------- top-k
// Report-summary page, section 9 (known limitations): at large batches a top-k truncation of
// the distribution is the named missing throughput optimisation.  With K > 0
// a row's statistics, draw and self-conditioning use its K largest logits,
// c_0..c_{K-1} by value descending, ties to the lower index:
//   m = l[c_0] (the argmax), z_i = l[c_i] - m, e_i = E(z_i), S and A the
//   sums of e_i and e_i * z_i in candidate order, H = max(0, L(S) - A / S),
//   pmax = 1 / S, draw: first running sum of w_i = E(z_i / T) above u * total
//   (u from Philox word 0), else the last positive; weights p_i = e_i / S.
// Finding the K largest without a full pass: with t the K-th largest of the
// row's 64-entry slab maxima, at least K entries are >= t, so every top-K
// entry is >= t and lies in a slab whose maximum is >= t.  The candidates
// are the slabs above t and the lowest-index K slabs whose maximum equals t
// (entries equal to t rank by index); their entries >= t are sorted.

constexpr int TK_THR = 256;
constexpr int TK_KEYS = 8192;      // >= (2 * kTopKMax - 1) * 64, a power of two

// Order-preserving unsigned key of a float (-0 taken as +0, so keys of
// numbers are equal exactly when the values compare equal); every NaN takes
// the largest key, above +inf, so NaN ranks above every number and NaNs tie
// (then the lower index first).
__device__ __forceinline__ uint32_t okey(float v) {
    if (v != v) return 0xFFFFFFFFu;
    const uint32_t u = v == 0.0f ? 0u : __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(TK_THR) void sample_topk_kernel(SampleArgs a) {
    extern __shared__ __align__(16) unsigned char tk_sm[];
    const int nslab = cdiv(a.V, 64);
    uint64_t* keys = reinterpret_cast<uint64_t*>(tk_sm);                 // [TK_KEYS]
    float* cval = reinterpret_cast<float*>(keys + TK_KEYS);              // [2 kTopKMax][64]
    uint32_t* skey = reinterpret_cast<uint32_t*>(cval + 2 * kTopKMax * 64);   // [nslab]
    __shared__ uint32_t hist[TK_THR / 64][256];   // one histogram per wave
    __shared__ int gt_list[kTopKMax], eq_list[kTopKMax];
    __shared__ int ctl[4];               // selected digit, remaining rank, #gt, #eq (capped)
    __shared__ uint32_t red[2][TK_THR / 64];
    __shared__ unsigned int nf;
    __shared__ int cidx[kTopKMax];
    __shared__ float cz[kTopKMax], ce[kTopKMax], cw[kTopKMax];
    __shared__ float sS;

    const long rowid = blockIdx.x;
    const int b = (int)(rowid / a.N), i = (int)(rowid % a.N);
    if (a.stop[b]) return;
    const float* row = a.logits + rowid * (long)a.V;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = min(a.top_k, a.V);

    // 1. slab maxima as keys, and their smallest and largest key
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
    if (a.rowmax) {
        const float* rm = a.rowmax + rowid * (long)nslab;
        for (int sl = tid; sl < nslab; sl += TK_THR) {
            const uint32_t k = okey(rm[sl]);
            skey[sl] = k;
            lmin = min(lmin, k);
            lmax = max(lmax, k);
        }
    } else {
        for (int sl = tid; sl < nslab; sl += TK_THR) {
            const int k0 = sl * 64, k1 = min(a.V, k0 + 64);
            float mx = row[k0];
            for (int k = k0 + 1; k < k1; ++k) mx = max_nan(mx, row[k]);
            const uint32_t k = okey(mx);
            skey[sl] = k;
            lmin = min(lmin, k);
            lmax = max(lmax, k);
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        lmin = min(lmin, (uint32_t)__shfl_xor((int)lmin, o, 64));
        lmax = max(lmax, (uint32_t)__shfl_xor((int)lmax, o, 64));
    }
    if (lane == 0) {
        red[0][wave] = lmin;
        red[1][wave] = lmax;
    }
    __syncthreads();
    uint32_t kmin = red[0][0], kmax = red[1][0];
#pragma unroll
    for (int w = 1; w < TK_THR / 64; ++w) {
        kmin = min(kmin, red[0][w]);
        kmax = max(kmax, red[1][w]);
    }

    // 2. t = the K-th largest slab key: radix select over the bits below the
    // keys' common prefix, 8 at a time (fewer slabs than K: every slab is a
    // candidate, t below every key)
    uint32_t prefix = 0, pmask = 0;
    int hi = 0;
    if (K <= nslab) {
        const uint32_t diff = kmin ^ kmax;
        hi = diff ? 32 - __builtin_clz(diff) : 0;       // bits still to decide
        pmask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
        prefix = kmax & pmask;
    }
    int need = K;
#pragma unroll 1
    while (hi > 0) {
        const int w = hi < 8 ? hi : 8;
        const int shift = hi - w;
        const uint32_t dmask = (1u << w) - 1u;
        for (int x = tid; x < (TK_THR / 64) * 256; x += TK_THR) (&hist[0][0])[x] = 0u;
        __syncthreads();
        for (int sl = tid; sl < nslab; sl += TK_THR) {
            const uint32_t k = skey[sl];
            if ((k & pmask) == prefix) atomicAdd(&hist[wave][(k >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds digits 4l .. 4l+3; counts from the top digit down
            uint32_t cnt[4], tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cnt[q] = 0;
#pragma unroll
                for (int ww = 0; ww < TK_THR / 64; ++ww) cnt[q] += hist[ww][4 * lane + q];
                tot += cnt[q];
            }
            uint32_t suf = tot;                       // lanes >= l
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = (uint32_t)__shfl_down((int)suf, o, 64);
                if (lane + o < 64) suf += t;
            }
            uint32_t acc = suf - tot;                 // lanes > l: larger digits
#pragma unroll
            for (int q = 3; q >= 0; --q) {
                if (acc < (uint32_t)need && acc + cnt[q] >= (uint32_t)need) {
                    ctl[0] = 4 * lane + q;
                    ctl[1] = need - (int)acc;
                }
                acc += cnt[q];
            }
        }
        __syncthreads();
        prefix |= (uint32_t)ctl[0] << shift;
        pmask |= dmask << shift;
        need = ctl[1];
        hi = shift;
        __syncthreads();
    }

    // 3. candidate slabs, in slab order: all above t, the first K equal to t
    if (wave == 0) {
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        int ngt = 0, neq = 0;
        for (int base = 0; base < nslab; base += 64) {
            const int sl = base + lane;
            const uint32_t k = sl < nslab ? skey[sl] : 0u;
            const bool gt = sl < nslab && k > prefix, eq = sl < nslab && k == prefix;
            const uint64_t mg = __ballot(gt), me = __ballot(eq);
            const int rg = __popcll(mg & below), re = __popcll(me & below);
            if (gt && ngt + rg < kTopKMax) gt_list[ngt + rg] = sl;
            if (eq && neq + re < K) eq_list[neq + re] = sl;
            ngt += __popcll(mg);
            neq += __popcll(me);
        }
        if (lane == 0) {
            ctl[2] = min(ngt, kTopKMax);    // at most K - 1 slabs exceed t
            ctl[3] = min(neq, K);
            nf = 0;
        }
    }
    __syncthreads();
    const int ngt = ctl[2], ncand = ctl[2] + ctl[3];

    // 4. the candidate slabs' logits into LDS (16 threads a slab, all loads
    // issued before any is used), then their entries >= t as (key, reversed
    // index) pairs
    const bool vec = (a.V & 3) == 0;
#pragma unroll 8
    for (int base = 0; base < 2 * kTopKMax; base += TK_THR / 16) {
        const int j = base + (tid >> 4);
        if (j < ncand) {
            const int sl = j < ngt ? gt_list[j] : eq_list[j - ngt];
            const int q = (tid & 15) * 4;
            const int k = sl * 64 + q;
            float4 v;
            if (vec && k + 3 < a.V) {
                v = *reinterpret_cast<const float4*>(row + k);
            } else {
                v.x = k < a.V ? row[k] : 0.0f;
                v.y = k + 1 < a.V ? row[k + 1] : 0.0f;
                v.z = k + 2 < a.V ? row[k + 2] : 0.0f;
                v.w = k + 3 < a.V ? row[k + 3] : 0.0f;
            }
            *reinterpret_cast<float4*>(cval + j * 64 + q) = v;
        }
    }
    __syncthreads();
    for (int e = tid; e < ncand * 64; e += TK_THR) {
        const int j = e >> 6;
        const int sl = j < ngt ? gt_list[j] : eq_list[j - ngt];
        const int k = sl * 64 + (e & 63);
        if (k < a.V) {
            const uint32_t kv = okey(cval[e]);
            if (kv >= prefix) {
                const unsigned int pos = atomicAdd(&nf, 1u);
                keys[pos] = ((uint64_t)kv << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)k);
            }
        }
    }
    __syncthreads();

    // 5. bitonic sort, descending (larger value first, then lower index)
    int P = 64;
    while (P < (int)nf) P <<= 1;
    for (int e = (int)nf + tid; e < P; e += TK_THR) keys[e] = 0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int x = tid; x < P; x += TK_THR) {
                const int y = x ^ stride;
                if (y > x) {
                    const bool desc = (x & size) == 0;
                    const uint64_t kx = keys[x], ky = keys[y];
                    if ((kx < ky) == desc) {
                        keys[x] = ky;
                        keys[y] = kx;
                    }
                }
            }
            __syncthreads();
        }
    }

    // 6. the K candidates: weights in parallel, the sums in order
    if (tid < K) cidx[tid] = (int)(0xFFFFFFFFu - (uint32_t)keys[tid]);
    __syncthreads();
    const float m = row[cidx[0]];
    if (tid < K) {
        const float z = row[cidx[tid]] - m;
        cz[tid] = z;
        ce[tid] = dexp(z);
        cw[tid] = dexp(z * a.inv_t);
    }
    __syncthreads();
    if (tid == 0) {
        float S = 0.0f, A = 0.0f;
        for (int c = 0; c < K; ++c) {
            S = S + ce[c];
            const float ez = ce[c] * cz[c];
            A = A + ez;
        }
        sS = S;
        if (!a.list_only) {
            uint64_t o[4];
            philox((uint64_t)a.step, (uint64_t)b, (uint64_t)i, 0ull, a.seed, 0ull, o);
            float H = dlog(S) - A / S;
            H = H > 0.0f ? H : (H != H ? H : 0.0f);  // NaN (non-finite logits) stays NaN
            float* st = a.stats + rowid * 4;
            st[0] = m;
            st[1] = S;
            st[2] = H;
            st[3] = 1.0f / S;
            a.newmax[rowid] = cidx[0];
            a.y[rowid] = cidx[pick_seq(cw, K, uniform01(o[0]))];
            a.r[rowid] = uniform_token(o[1], a.V);
        }
    }
    __syncthreads();
    if (a.tk_idx && tid < K) {
        a.tk_idx[rowid * K + tid] = cidx[tid];
        a.tk_p[rowid * K + tid] = ce[tid] / sS;
    }
}

// One workgroup per canvas: lock rule, renoise, stability and stop.
__global__ __launch_bounds__(1024) void sample_canvas_kernel(SampleArgs a) {
    const int b = blockIdx.x;
    if (a.stop[b]) {
        if (threadIdx.x == 0 && a.host_stop) a.host_stop[b] = a.stop[b];
        return;
    }
    __shared__ uint64_t keys[1024];
    __shared__ float Hs[1024];
    __shared__ uint8_t lk[1024];
    const int tid = threadIdx.x;
    const int N = a.N;
    const long base = (long)b * N;
    int npow = 1;
    while (npow < N) npow <<= 1;
    for (int i = tid; i < npow; i += blockDim.x) {
        if (i < N) {
            const float H = a.stats[(base + i) * 4 + 2];
            Hs[i] = H;
            keys[i] = ((uint64_t)__float_as_uint(H) << 32) | (uint32_t)i;
            lk[i] = a.lock_rule == 0 ? (a.stats[(base + i) * 4 + 3] > a.theta ? 1 : 0) : 0;
        } else {
            keys[i] = ~0ull;
        }
    }
    // a NaN entropy means a non-finite logit in that row: the canvas is
    // reported (stop 2) and left as it was
    int nan_here = 0;
    for (int i = tid; i < N; i += blockDim.x) nan_here |= Hs[i] != Hs[i];
    const int bad = __syncthreads_or(nan_here);
    if (bad) {
        if (tid == 0) {
            a.stop[b] = 2;
            if (a.host_stop) a.host_stop[b] = 2;
            if (a.trace) {
                a.trace[2 * b] = __builtin_nanf("");
                a.trace[2 * b + 1] = 0.0f;
            }
            if (a.nstop && atomicAdd(a.nstop, 1) + 1 == a.B) *a.halt = 1;
        }
        return;
    }
    if (a.lock_rule == 1) {
        // bitonic sort of (H, index); H >= 0 so its bits order like the value
        for (int size = 2; size <= npow; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < npow; i += blockDim.x) {
                    const int p = i ^ stride;
                    if (p > i) {
                        const bool up = (i & size) == 0;
                        const uint64_t ki = keys[i], kp = keys[p];
                        if ((ki > kp) == up) {
                            keys[i] = kp;
                            keys[p] = ki;
                        }
                    }
                }
                __syncthreads();
            }
        }
        if (tid == 0) {
            float acc = 0.0f;
            for (int n = 0; n < N; ++n) {
                const int i = (int)(uint32_t)keys[n];
                const float H = Hs[i];
                if (acc + H <= a.theta) {
                    lk[i] = 1;
                    acc = acc + H;
                } else {
                    break;
                }
            }
        }
        __syncthreads();
    }
    int same = 1;
    for (int i = tid; i < N; i += blockDim.x) {
        const int am = a.newmax[base + i];
        if (a.argmax[base + i] != am) same = 0;
        a.argmax[base + i] = am;
        a.lock[base + i] = lk[i];
        a.canvas[base + i] = lk[i] ? a.y[base + i] : a.r[base + i];
    }
    const int stable = __syncthreads_and(same) && a.step > 0;
    if (tid == 0) {
        float sumH = 0.0f;
        for (int i = 0; i < N; ++i) sumH = sumH + Hs[i];
        const float meanH = sumH / (float)N;
        if (a.trace) {
            int nl = 0;
            for (int i = 0; i < N; ++i) nl += lk[i];
            a.trace[2 * b] = meanH;
            a.trace[2 * b + 1] = (float)nl;
        }
        int st = (meanH < a.tau) && (!a.require_stable || stable);
        if (a.step + 1 >= a.max_steps) st = 1;
        a.stop[b] = st;
        if (a.host_stop) a.host_stop[b] = st;
        // the last sequence to stop raises the halt flag
        if (st && a.nstop && atomicAdd(a.nstop, 1) + 1 == a.B) *a.halt = 1;
    }
}

__global__ __launch_bounds__(256) void canvas_init_kernel(uint64_t seed, int block, int N, int V,
                                                          int32_t* canvas, long total) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int b = (int)(idx / N), i = (int)(idx % N);
    uint64_t o[4];
    philox((uint64_t)block, (uint64_t)b, (uint64_t)i, 1ull, seed, 0ull, o);
    canvas[idx] = uniform_token(o[0], V);
}

// ------------------------------------------------- training-side forward
// Report-summary page, sections 1 and 3: training replaces a random share
// of a text's tokens (0 to 100 %) and scores the prediction at the
// originals.  Position (b, i) is replaced when the uniform of Philox word 0
// (counter (step, b, i, 2)) is below its canvas's rate, by the uniform
// token of word 1.
__global__ __launch_bounds__(256) void corrupt_kernel(uint64_t seed, int step, int N, int V,
                                                      const float* __restrict__ rate,
                                                      const int32_t* __restrict__ clean,
                                                      int32_t* __restrict__ out, long total) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int b = (int)(idx / N), i = (int)(idx % N);
    uint64_t o[4];
    philox((uint64_t)step, (uint64_t)b, (uint64_t)i, 2ull, seed, 0ull, o);
    out[idx] = uniform01(o[0]) < rate[b] ? uniform_token(o[1], V) : clean[idx];
}

// The mean loss: one lane adds the rows in order (the definition is a
// sequential binary32 sum), the other lanes prefetch nothing; rows are few.
__global__ __launch_bounds__(64) void mean_seq_kernel(const float* __restrict__ loss, int rows,
                                                      float* __restrict__ mean) {
    if (threadIdx.x != 0) return;
    float acc = 0.0f;
    for (int r = 0; r < rows; ++r) acc = acc + loss[r];
    mean[0] = acc / (float)rows;
}

// ------------------------------------------------------- greedy (AR mode)
// Greedy decoding takes each row's largest logit, ties to the lower index.
// A NaN ranks above every number (the first NaN of a row is its choice, as
// numpy's argmax has it), so a non-finite row shows in the decoded token
// stream instead of being skipped.

// (value, index) maximum: (v, i) beats (bv, bi) when v > bv, or when v is
// NaN and bv is not, or when they are equal (or both NaN) and i < bi.
__device__ __forceinline__ void amax_take(float v, int i, float& bv, int& bi) {
    const bool vn = v != v, bn = bv != bv;
    if ((vn && !bn) || v > bv || ((v == bv || (vn && bn)) && i < bi)) {
        bv = v;
        bi = i;
    }
}

// Block-wide (value, index) reduction of AM_THR threads; the result in
// every thread.
template <int NT>
__device__ __forceinline__ void amax_block(float& bv, int& bi) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        amax_take(ov, oi, bv, bi);
    }
    __shared__ float wv[NT / 64];
    __shared__ int wi[NT / 64];
    if ((threadIdx.x & 63) == 0) {
        wv[threadIdx.x >> 6] = bv;
        wi[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    bv = wv[0];
    bi = wi[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) amax_take(wv[w], wi[w], bv, bi);
}

// One workgroup per row: four float4 loads in flight per thread.
constexpr int AM_THR = 1024;
__global__ __launch_bounds__(AM_THR) void argmax_rows_kernel(const float* __restrict__ x, int V,
                                                             int32_t* __restrict__ out,
                                                             long out_stride) {
    const long row = blockIdx.x;
    const float* r = x + row * (long)V;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    if ((V & 3) == 0) {
        const float4* r4 = reinterpret_cast<const float4*>(r);
        const int n4 = V >> 2;
        for (int j0 = threadIdx.x; j0 < n4; j0 += 4 * AM_THR) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * AM_THR;
                v[u] = j < n4 ? r4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (j0 + u * AM_THR >= n4) continue;    // past the row: no candidate
                const int i = 4 * (j0 + u * AM_THR);
                amax_take(v[u].x, i, bv, bi);
                amax_take(v[u].y, i + 1, bv, bi);
                amax_take(v[u].z, i + 2, bv, bi);
                amax_take(v[u].w, i + 3, bv, bi);
            }
        }
    } else {
        for (int j = threadIdx.x; j < V; j += AM_THR) amax_take(r[j], j, bv, bi);
    }
    amax_block<AM_THR>(bv, bi);
    if (threadIdx.x == 0) out[row * out_stride] = bi == 0x7FFFFFFF ? 0 : bi;
}

// From the head's 64-column slab maxima (V % 64 == 0, a NaN member makes its
// slab's maximum NaN): the first slab whose maximum is the row's largest,
// then the first entry of that slab equal to it (a NaN, if it is NaN).
// Every earlier slab's maximum is smaller, so this is the first index of the
// row's maximum.
__global__ __launch_bounds__(256) void argmax_slabs_kernel(const float* __restrict__ x,
                                                           const float* __restrict__ rowmax, int V,
                                                           int32_t* __restrict__ out,
                                                           long out_stride) {
    const long row = blockIdx.x;
    const int nslab = V >> 6;
    const float* rm = rowmax + row * (long)nslab;
    float bv = -INFINITY;
    int bs = 0x7FFFFFFF;
    // eight slab maxima in flight per thread before they are compared (the
    // (value, lowest index) maximum does not depend on the visiting order)
    int sl = threadIdx.x;
    for (; sl + 7 * 256 < nslab; sl += 8 * 256) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = rm[sl + q * 256];
#pragma unroll
        for (int q = 0; q < 8; ++q) amax_take(v[q], sl + q * 256, bv, bs);
    }
    for (; sl < nslab; sl += 256) amax_take(rm[sl], sl, bv, bs);
    amax_block<256>(bv, bs);
    if (threadIdx.x < 64) {
        int idx = 0;
        if (bs != 0x7FFFFFFF) {
            const float v = x[row * (long)V + (long)bs * 64 + threadIdx.x];
            const uint64_t hit = __ballot(v == bv || (v != v && bv != bv));
            idx = bs * 64 + (hit ? __builtin_ctzll(hit) : 0);
        }
        if (threadIdx.x == 0) out[row * out_stride] = idx;
    }
}

}  // namespace

hipError_t corrupt(uint64_t seed, int step, int B, int N, int V, const float* rate,
                   const int32_t* clean, int32_t* out, hipStream_t st) {
    const long total = (long)B * N;
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(corrupt_kernel, dim3((unsigned)cdiv((int)total, 256)), dim3(256), 0, st,
                       seed, step, N, V, rate, clean, out, total);
    return hipGetLastError();
}

hipError_t mean_seq(const float* loss, int rows, float* mean, hipStream_t st) {
    if (rows <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mean_seq_kernel, dim3(1), dim3(64), 0, st, loss, rows, mean);
    return hipGetLastError();
}

hipError_t argmax_rows(const float* logits, int rows, int V, int32_t* out, long out_stride,
                       hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (V <= 0 || ((uintptr_t)logits & 15)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(argmax_rows_kernel, dim3(rows), dim3(AM_THR), 0, st, logits, V, out,
                       out_stride);
    return hipGetLastError();
}

hipError_t argmax_slabs(const float* logits, const float* rowmax, int rows, int V, int32_t* out,
                        long out_stride, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (V <= 0 || V % 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL(argmax_slabs_kernel, dim3(rows), dim3(256), 0, st, logits, rowmax, V, out,
                       out_stride);
    return hipGetLastError();
}

hipError_t sample_update(const SampleArgs& a, hipStream_t st) {
    if (a.B <= 0 || a.N <= 0) return hipSuccess;
    if (a.stats_only && (a.top_k || a.probs || (a.loss && !a.target))) return hipErrorInvalidValue;
    if (a.top_k > 0) {
        const int nslab = cdiv(a.V, 64);
        if (a.top_k > kTopKMax || a.top_k > a.V || (a.rowmax && a.rowmax_n != nslab) ||
            (a.tk_idx == nullptr) != (a.tk_p == nullptr) || (a.list_only && !a.tk_idx))
            return hipErrorInvalidValue;
        const size_t lds = (size_t)TK_KEYS * 8 + (size_t)2 * kTopKMax * 64 * 4 + (size_t)nslab * 4;
        static bool tk_attr = false;
        if (!tk_attr) {
            hipError_t e = hipFuncSetAttribute((const void*)sample_topk_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)(TK_KEYS * 8 + 2 * kTopKMax * 64 * 4 + 8192 * 4));
            if (e != hipSuccess) return e;
            tk_attr = true;
        }
        hipLaunchKernelGGL(sample_topk_kernel, dim3(a.B * a.N), dim3(TK_THR), lds, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.list_only) return e;
        hipLaunchKernelGGL(sample_canvas_kernel, dim3(a.B), dim3(1024), 0, st, a);
        return hipGetLastError();
    }
    if (a.probs && (a.V % 128 || !a.rowmax || a.rowmax_n < 1 || ((uintptr_t)a.logits & 15) ||
                    ((uintptr_t)a.probs & 7)))
        return hipErrorInvalidValue;
    const int nt = cdiv(a.V, TILE);
    const size_t lds = (size_t)2 * nt * NLANE * sizeof(float);
    static bool attr_set[3] = {false, false, false};
    const bool vec = (a.V % 4) == 0;
    const int which = a.probs ? 2 : (vec ? 1 : 0);
    const void* kerns[3] = {(const void*)sample_row_kernel<false, false>,
                            (const void*)sample_row_kernel<true, false>,
                            (const void*)sample_row_kernel<true, true>};
    if (!attr_set[which]) {
        hipError_t e = hipFuncSetAttribute(kerns[which], hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(2 * 8 * NLANE * sizeof(float)));
        if (e != hipSuccess) return e;
        attr_set[which] = true;
    }
    if (a.probs)
        hipLaunchKernelGGL((sample_row_kernel<true, true>), dim3(a.B * a.N), dim3(NTHR), lds, st, a);
    else if (vec)
        hipLaunchKernelGGL((sample_row_kernel<true, false>), dim3(a.B * a.N), dim3(NTHR), lds, st, a);
    else
        hipLaunchKernelGGL((sample_row_kernel<false, false>), dim3(a.B * a.N), dim3(NTHR), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.stats_only) return e;
    hipLaunchKernelGGL(sample_canvas_kernel, dim3(a.B), dim3(1024), 0, st, a);
    return hipGetLastError();
}

hipError_t selfcond_probs(const float* logits, const float* stats, uint16_t* out, int rows, int V,
                          const int32_t* halt, int tiled, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (V % 4 || (tiled && V % 64)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(selfcond_probs_kernel, dim3(rows, 4 * cdiv(V, TILE)), dim3(256), 0, st, logits,
                       stats, out, V, halt, tiled);
    return hipGetLastError();
}

hipError_t canvas_init(uint64_t seed, int block, int B, int N, int V, int32_t* canvas,
                       hipStream_t st) {
    const long total = (long)B * N;
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(canvas_init_kernel, dim3((unsigned)cdiv((int)total, 256)), dim3(256), 0, st,
                       seed, block, N, V, canvas, total);
    return hipGetLastError();
}

}  // namespace dg
