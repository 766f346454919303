// Grouped-query attention over the KV cache on gfx950 MFMA.
//
// The denoiser's canvas queries see every cached context key and every
// canvas key (no mask); the encoder's queries see keys up to their own
// position (causal).  Report-summary page (animattoys.com), section 2;
// youleyou.com article, "Architecture basis".
//
// Three kernels: attn3_kernel (bf16, head dim 128, the canvas: 32 queries a
// wave on the 32x32x16 MFMA), attn2_kernel (bf16, head dim 128, causal: the
// prompt encode and decode steps) and attn_kernel (other shapes, fp32).
// In attn_kernel and attn2_kernel a wave owns 16 queries of one query head;
// the four waves of a workgroup share one KV head, so each K/V tile staged
// in LDS serves all of them.
// Scores are computed transposed, S^T = K Q^T, so that a lane holds 8 keys of
// ONE query: the online-softmax state (max, sum, rescale) is lane-local
// except for one max across the 4 lanes of a query, and the probabilities
// already sit in the B-operand layout of O^T = V^T P^T.  Long key ranges are
// split across workgroups and merged by a second kernel.
#include <algorithm>
#include <cstdlib>

#include "common.h"
#include "kernels.h"
#include "lds_ring.h"

namespace dg {

namespace {

constexpr int KT = 32;  // keys per tile
constexpr float LOG2E = 1.4426950408889634f;

template <typename T> struct AttnLds {
    static constexpr int KPAD = 16 / (int)sizeof(T);  // K row padding (elements)
    static constexpr int VPAD = 16 / (int)sizeof(T);  // V^T row padding (elements)
    static constexpr int CE = 16 / (int)sizeof(T);    // elements per 16-byte chunk
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Workgroup barrier that waits only for this wave's LDS traffic (global
// loads in flight stay in flight).
__device__ __forceinline__ void attn_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
}

// V^T fragment: row d, keys {4g..4g+3} and {16+4g..16+4g+3}.
__device__ __forceinline__ void load_vt(Frag<bf16_t>& f, const bf16_t* row, int g4) {
    uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * g4);
    uint2 hi = *reinterpret_cast<const uint2*>(row + 16 + 4 * g4);
    f.v = make_uint4(lo.x, lo.y, hi.x, hi.y);
}
__device__ __forceinline__ void load_vt(Frag<float>& f, const float* row, int g4) {
    f.lo = *reinterpret_cast<const float4*>(row + 4 * g4);
    f.hi = *reinterpret_cast<const float4*>(row + 16 + 4 * g4);
}

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
    if (a.halt && *a.halt) return;
    using L = AttnLds<T>;
    constexpr int KROW = DH + L::KPAD;
    constexpr int VROW = KT + L::VPAD;
    constexpr int NQF = DH / 32;   // Q fragments (k-steps over dh)
    constexpr int NOT = DH / 16;   // O^T tiles over dh
    __shared__ __align__(16) T Ks[KT * KROW];
    // bf16: V kept as it is in the cache, [key][dh] with rows padded to
    // DH + 16 (the four key rows one transposed read touches fall in
    // distinct banks), read transposed by ds_read_b64_tr_b16; fp32: V^T
    // written element by element
    constexpr bool TRV = sizeof(T) == 2;
    constexpr int VRROW = DH + 16;
    __shared__ __align__(16) T Vt[TRV ? KT * VRROW : DH * VROW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int G = a.Hq / a.Hkv;
    const int nqt = cdiv(a.n, 16);
    const int kvh = blockIdx.y;
    const int b = blockIdx.z / a.splits, split = blockIdx.z % a.splits;

    const int unit = blockIdx.x * 4 + wave;
    const bool wvalid = unit < G * nqt;
    const int qt = wvalid ? unit / G : 0;
    const int h = kvh * G + (wvalid ? unit % G : 0);
    const int qi = qt * 16 + r16;          // this lane's query (within the n new tokens)
    const bool qvalid = wvalid && qi < a.n;
    const long qrow = (long)b * a.n + (qvalid ? qi : 0);
    const int qpos = a.pos0 + qi;

    // key range of this split; causal: up to the last query of the workgroup
    int kb = split * a.split_len;
    int ke = min(a.kv_len, kb + a.split_len);
    if (a.causal) {
        int last_unit = min(blockIdx.x * 4 + 3, G * nqt - 1);
        int last_q = min(a.n - 1, (last_unit / G) * 16 + 15);
        ke = min(ke, a.pos0 + last_q + 1);
    }

    // Q fragments (B operand of S^T = K Q^T)
    Frag<T> qf[NQF];
    {
        const T* Q = reinterpret_cast<const T*>(a.q) + qrow * (long)a.Hq * DH + (long)h * DH;
#pragma unroll
        for (int s = 0; s < NQF; ++s) {
            if (qvalid) load_frag(qf[s], Q + s * 32 + g4 * 8);
            else zero_frag(qf[s]);
        }
    }

    f32x4_t o[NOT];
#pragma unroll
    for (int i = 0; i < NOT; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -1e30f, l_run = 0.f;
    const float qscale = LOG2E / sqrtf((float)DH);

    const T* Kc = reinterpret_cast<const T*>(a.kc) + ((long)b * a.Hkv + kvh) * (long)a.cap * DH;
    const T* Vc = reinterpret_cast<const T*>(a.vc) + ((long)b * a.Hkv + kvh) * (long)a.cap * DH;
    constexpr int CHUNKS = KT * DH / L::CE;   // 16-byte chunks per K (or V) tile
    constexpr int NC = CHUNKS / 256;          // per thread
    static_assert(NC >= 1 && CHUNKS % 256 == 0, "tile chunks must split over the workgroup");

    // This thread's chunks of a tile are loaded one tile ahead into
    // registers (kr, vr): the loads of tile t+1 are in flight while tile t
    // is multiplied.  The barriers wait only for LDS traffic, so those loads
    // stay outstanding across them; their first use (the LDS store of the
    // next pass) waits for them.
    uint4 kr[NC], vr[NC];
#define ATT_GLOAD(K0)                                                                         \
    _Pragma("unroll") for (int c = 0; c < NC; ++c) {                                          \
        const int ch = tid + c * 256;                                                         \
        const int key = ch / (DH / L::CE);                                                    \
        const int d0 = (ch % (DH / L::CE)) * L::CE;                                           \
        kr[c] = make_uint4(0, 0, 0, 0);                                                       \
        vr[c] = kr[c];                                                                        \
        if ((K0) + key < ke) {                                                                \
            kr[c] = *reinterpret_cast<const uint4*>(Kc + (long)((K0) + key) * DH + d0);       \
            vr[c] = *reinterpret_cast<const uint4*>(Vc + (long)((K0) + key) * DH + d0);       \
        }                                                                                     \
    }
    if (kb < ke) ATT_GLOAD(kb);
    for (int k0 = kb; k0 < ke; k0 += KT) {
        attn_barrier();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int ch = tid + c * 256;
            const int key = ch / (DH / L::CE);
            const int d0 = (ch % (DH / L::CE)) * L::CE;
            *reinterpret_cast<uint4*>(&Ks[key * KROW + d0]) = kr[c];
            if constexpr (TRV) {
                *reinterpret_cast<uint4*>(&Vt[key * VRROW + d0]) = vr[c];
            } else {
                const T* vp = reinterpret_cast<const T*>(&vr[c]);
#pragma unroll
                for (int i = 0; i < L::CE; ++i) Vt[(d0 + i) * VROW + key] = vp[i];
            }
        }
        attn_barrier();
        if (k0 + KT < ke) ATT_GLOAD(k0 + KT);

        // S^T for 32 keys: lane holds keys kt*16 + 4*g4 + e of query r16
        f32x4_t sc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NQF; ++s) {
                Frag<T> kf;
                load_frag(kf, &Ks[(kt * 16 + r16) * KROW + s * 32 + g4 * 8]);
                mma(sc[kt], kf, qf[s]);
            }
        }
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = k0 + kt * 16 + 4 * g4 + e;
                bool ok = key < ke && (!a.causal || key <= qpos);
                float v = ok ? sc[kt][e] * qscale : -INFINITY;
                x[kt * 4 + e] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float corr = exp2f(m_run - m_new);
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = exp2f(x[i] - m_new);
            psum += p[i];
        }
        l_run = l_run * corr + psum;
        m_run = m_new;
        Frag<T> pf;
        frag_from_f(pf, p);
#pragma unroll
        for (int dt = 0; dt < NOT; ++dt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[dt][e] *= corr;
            Frag<T> vf;
            if constexpr (TRV) {
                // lane j of a 16-lane group gives the address of keys
                // 4*g4 + j/4 (+16), dh dt*16 + 4*(j%4) .. +3; lane 4a+b then
                // receives dh dt*16 + 4a+b of keys 4*g4 + 0..3 (+16): row r16,
                // the same keys as its probabilities
                typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
                const T* vb = &Vt[(4 * g4 + (r16 >> 2)) * VRROW + dt * 16 + 4 * (r16 & 3)];
                const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb));
                const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + 16 * VRROW));
                vf.v = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                  __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y);
            } else {
                load_vt(vf, &Vt[(dt * 16 + r16) * VROW], g4);
            }
            mma(o[dt], vf, pf);
        }
    }

#undef ATT_GLOAD

    // lane holds O^T[d = dt*16 + 4*g4 + e][query r16]
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot = l_tot + __shfl_xor(l_tot, 32, 64);
    if (!qvalid) return;
    if (a.splits == 1) {
        T* out = reinterpret_cast<T*>(a.out) + qrow * (long)a.Hq * DH + (long)h * DH;
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
        for (int dt = 0; dt < NOT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) out[dt * 16 + 4 * g4 + e] = Elt<T>::from_f(o[dt][e] * inv);
    } else {
        const long base = ((long)split * a.B * a.n + qrow) * a.Hq + h;
        float* po = a.part_o + base * DH;
#pragma unroll
        for (int dt = 0; dt < NOT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) po[dt * 16 + 4 * g4 + e] = o[dt][e];
        if (g4 == 0) {
            a.part_ml[base * 2 + 0] = m_run;
            a.part_ml[base * 2 + 1] = l_tot;
        }
    }
}

// ------------------------------------------------------------------------
// bf16, head dim 128: the same attention as attn_kernel, organised so that
// the matrix cores rather than the softmax bookkeeping set the pace.
//
//   * A wave owns 16 queries of HPW query heads of one KV group (HPW = 1:
//     four workgroups of 128 registers per wave fit on a CU, and that
//     occupancy hides the LDS and barrier latency better than two heads per
//     wave at half the occupancy; measured 0.107 against 0.121-0.127 ms at
//     33 024 keys).
//   * K and V tiles of 32 keys arrive by direct-to-LDS loads
//     (global_load_lds, no register staging) in a ring of two slots: the
//     next tile loads while this one is multiplied; the barrier waits for
//     LDS traffic only.
//   * Each 256-byte key row keeps its sixteen 16-byte chunks XOR-swizzled,
//     with one swizzle per operand, each measured on gfx950 to read at the
//     rate of a linear read: K rows hold chunk c in slot c ^ (r % 16) for
//     the fragment reads (16 rows, one chunk each; about 220 B a clock and
//     CU, against 117 with the V swizzle), V rows hold it in slot c ^ sw2(r)
//     for the transposing reads (4 rows x 32 bytes per 16 lanes; 192 B a
//     clock, against 118 with the K swizzle).
//   * Q is scaled by log2(e)/sqrt(dh) once, when its fragments are loaded,
//     so a score is already the exponent of 2 the softmax needs.
//   * The running maximum moves only when a tile's maximum exceeds it by
//     more than RESCALE_T (2^8 in the weights): O and the sums are then
//     rescaled; otherwise probabilities are taken against the stale maximum,
//     which changes no result (every partial is a consistent (o, m, l)
//     triple) but takes the rescale and the cross-lane maximum off the
//     common path.
//   * Key masks run only on the tiles that need them (the last partial
//     tile; causal tiles that reach past the wave's first query).
constexpr int KT2 = 32;              // keys per tile
constexpr int RING2 = 2;             // LDS slots (K and V tile each)
constexpr int ROW2 = 256;            // bytes per key row (128 bf16)
constexpr int TILE2 = KT2 * ROW2;    // 8 KiB per K (or V) tile
constexpr int SLOT2 = 2 * TILE2;     // K then V
constexpr float RESCALE_T = 8.0f;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int sw2(int r) {
    r &= 15;
    return (2 * r + (r >> 3)) & 15;
}


__device__ __forceinline__ uint32_t scale_bf2(uint32_t w, float c) {
    const float lo = __uint_as_float(w << 16) * c;
    const float hi = __uint_as_float(w & 0xFFFF0000u) * c;
    return pack_bf2(lo, hi);
}

template <int HPW>
__global__ __launch_bounds__(256, 4) void attn2_kernel(AttnArgs a) {
    if (a.halt && *a.halt) return;
    constexpr int DH = 128;
    __shared__ __align__(1024) unsigned char ring[RING2 * SLOT2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int G = a.Hq / a.Hkv;
    const int hg = G / HPW;                  // head groups of one KV head
    const int nqt = cdiv(a.n, 16);
    const int units = nqt * hg;
    // block -> (key range group, workgroup in it).  Blocks go to the eight
    // XCDs in turn; when the groups (KV head, sequence, key range) come in
    // eights, the workgroups of one group all land on one XCD, so each K/V
    // tile is fetched into one L2 and read from there by all of them.
    const int nx = cdiv(units, 4);
    const int ngroups = a.Hkv * a.B * a.splits;
    int bx, grp;
    if (ngroups % 8 == 0) {
        const int slot = blockIdx.x >> 3;
        bx = slot % nx;
        grp = (slot / nx) * 8 + (blockIdx.x & 7);
    } else {
        bx = blockIdx.x % nx;
        grp = blockIdx.x / nx;
    }
    const int kvh = grp % a.Hkv;
    const int b = (grp / a.Hkv) / a.splits, split = (grp / a.Hkv) % a.splits;
    const int unit = bx * 4 + wave;
    const bool wvalid = unit < units;
    const int qt = wvalid ? unit / hg : 0;
    const int h0 = kvh * G + (wvalid ? (unit % hg) * HPW : 0);
    const int qi = qt * 16 + r16;
    const bool qvalid = wvalid && qi < a.n;
    const long qrow = (long)b * a.n + (qvalid ? qi : 0);
    const int qpos = a.pos0 + qi;
    const int qpos_first = a.pos0 + qt * 16;

    int kb = split * a.split_len;
    int ke = min(a.kv_len, kb + a.split_len);
    if (a.causal) {
        const int last_unit = min(bx * 4 + 3, units - 1);
        const int last_q = min(a.n - 1, (last_unit / hg) * 16 + 15);
        ke = min(ke, a.pos0 + last_q + 1);
    }
    const int ntiles = ke > kb ? cdiv(ke - kb, KT2) : 0;

    // Q fragments, scaled so that a score is log2-e based
    const float qscale = LOG2E / sqrtf((float)DH);
    u32x4_t qf[HPW][4];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + qrow * (long)a.Hq * DH +
                          (long)(h0 + hh) * DH;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qvalid) v = *reinterpret_cast<const uint4*>(Q + s * 32 + g4 * 8);
            qf[hh][s] = u32x4_t{scale_bf2(v.x, qscale), scale_bf2(v.y, qscale),
                                scale_bf2(v.z, qscale), scale_bf2(v.w, qscale)};
        }
    }

    const bf16_t* Kc = reinterpret_cast<const bf16_t*>(a.kc) + ((long)b * a.Hkv + kvh) * (long)a.cap * DH;
    const bf16_t* Vc = reinterpret_cast<const bf16_t*>(a.vc) + ((long)b * a.Hkv + kvh) * (long)a.cap * DH;

    // direct-to-LDS fill: wave w writes 1 KiB blocks 2w and 2w+1 of each
    // tile; lane l of block q lands in row 4q + l/16, slot l%16, which holds
    // global chunk (l%16) ^ (row % 16) of a K row and (l%16) ^ sw2(row) of a
    // V row.  kof / vof: those chunks' byte offsets in a full tile; a partial
    // last tile clamps the row to the last valid key.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int frow[2];
    uint32_t kof[2], vof[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        frow[i] = 4 * (2 * wv + i) + (lane >> 4);
        kof[i] = frow[i] * ROW2 + (((lane & 15) ^ (frow[i] & 15)) << 4);
        vof[i] = frow[i] * ROW2 + (((lane & 15) ^ sw2(frow[i])) << 4);
    }
    const char* Kb = reinterpret_cast<const char*>(Kc);
    const char* Vb = reinterpret_cast<const char*>(Vc);
    auto issue = [&](int t) {
        const int k0_ = kb + t * KT2;
        unsigned char* sl_ = ring + (t % RING2) * SLOT2 + 2 * wv * 1024;
        const char* kt_ = Kb + (long)k0_ * ROW2;
        const char* vt_ = Vb + (long)k0_ * ROW2;
        if (k0_ + KT2 <= ke) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                __builtin_amdgcn_global_load_lds((glb_void*)(kt_ + kof[i]), (lds_void*)(sl_ + i * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((glb_void*)(vt_ + vof[i]), (lds_void*)(sl_ + TILE2 + i * 1024), 16, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t r_ = min(frow[i], ke - 1 - k0_) * ROW2;
                __builtin_amdgcn_global_load_lds((glb_void*)(kt_ + r_ + (kof[i] & (ROW2 - 1))), (lds_void*)(sl_ + i * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((glb_void*)(vt_ + r_ + (vof[i] & (ROW2 - 1))), (lds_void*)(sl_ + TILE2 + i * 1024), 16, 0, 0);
            }
        }
    };

    // fragment addresses within a slot (bytes): K for k-step s (subtile 1 at
    // +4096), V for dh tile dt (keys 16.. at +4096)
    uint32_t ka[4], va[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) ka[s] = r16 * ROW2 + (((4 * s + g4) ^ r16) << 4);
    {
        const int rv = 4 * g4 + (r16 >> 2);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            va[dt] = TILE2 + rv * ROW2 + (((2 * dt + ((r16 & 3) >> 1)) ^ sw2(rv)) << 4) +
                     8 * (r16 & 1);
    }
    const uint32_t ring0 = lds_addr(ring);

    // S^T = K Q^T of the tile in slot `sb`: lane holds keys kt*16 + 4*g4 + e
    // of query r16.  The K fragments are one asm block, so the compiler does
    // not wait for the direct-to-LDS loads of other slots before it.
    auto qk = [&](uint32_t sb, f32x4_t (&sc)[HPW][2]) {
        u32x4_t kf0, kf1, kf2, kf3, kf4, kf5, kf6, kf7;
        asm volatile(
            "ds_read_b128 %0, %8 offset:0\n ds_read_b128 %1, %9 offset:0\n"
            "ds_read_b128 %2, %10 offset:0\n ds_read_b128 %3, %11 offset:0\n"
            "ds_read_b128 %4, %8 offset:4096\n ds_read_b128 %5, %9 offset:4096\n"
            "ds_read_b128 %6, %10 offset:4096\n ds_read_b128 %7, %11 offset:4096\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(kf0), "=&v"(kf1), "=&v"(kf2), "=&v"(kf3), "=&v"(kf4), "=&v"(kf5), "=&v"(kf6),
              "=&v"(kf7)
            : "v"(sb + ka[0]), "v"(sb + ka[1]), "v"(sb + ka[2]), "v"(sb + ka[3])
            : "memory");
        const u32x4_t kf[2][4] = {{kf0, kf1, kf2, kf3}, {kf4, kf5, kf6, kf7}};
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                sc[hh][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    sc[hh][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, kf[kt][s]),
                        __builtin_bit_cast(bf16x8_t, qf[hh][s]), sc[hh][kt], 0, 0, 0);
            }
    };

    f32x4_t o[HPW][8];
    float m_run[HPW], l_run[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        m_run[hh] = -1e30f;
        l_run[hh] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[hh][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // softmax of the scores of the tile at keys k0.. (against the running
    // maximum, moved only past RESCALE_T) into bf16 probabilities, then
    // O^T += V^T P^T from the tile in slot `sb` (transposing V reads: keys
    // 4*g4 + 0..3 and +16)
    auto soft_pv = [&](uint32_t sb, int k0, f32x4_t (&sc)[HPW][2]) {
        const bool mask = (k0 + KT2 > ke) || (a.causal && k0 + KT2 - 1 > qpos_first);
        u32x4_t pf[HPW];
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            float x[8];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e) x[kt * 4 + e] = sc[hh][kt][e];
            if (mask) {
                const int key0 = k0 + 4 * g4;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = key0 + kt * 16 + e;
                        const bool ok = key < ke && (!a.causal || key <= qpos);
                        if (!ok) x[kt * 4 + e] = -INFINITY;
                    }
            }
            float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                             fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            if (__ballot(mx > m_run[hh] + RESCALE_T)) {
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float mn = fmaxf(m_run[hh], mx);
                const float corr = __builtin_amdgcn_exp2f(m_run[hh] - mn);
                l_run[hh] *= corr;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[hh][dt][e] *= corr;
                m_run[hh] = mn;
            }
            float p[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_run[hh]);
            l_run[hh] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            pf[hh] = u32x4_t{pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]), pack_bf2(p[4], p[5]),
                             pack_bf2(p[6], p[7])};
        }
        u32x2_t v0, v1, v2, v3, v4, v5, v6, v7, w0, w1, w2, w3, w4, w5, w6, w7;
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16 offset:0\n ds_read_b64_tr_b16 %1, %16 offset:4096\n"
            "ds_read_b64_tr_b16 %2, %17 offset:0\n ds_read_b64_tr_b16 %3, %17 offset:4096\n"
            "ds_read_b64_tr_b16 %4, %18 offset:0\n ds_read_b64_tr_b16 %5, %18 offset:4096\n"
            "ds_read_b64_tr_b16 %6, %19 offset:0\n ds_read_b64_tr_b16 %7, %19 offset:4096\n"
            "ds_read_b64_tr_b16 %8, %20 offset:0\n ds_read_b64_tr_b16 %9, %20 offset:4096\n"
            "ds_read_b64_tr_b16 %10, %21 offset:0\n ds_read_b64_tr_b16 %11, %21 offset:4096\n"
            "ds_read_b64_tr_b16 %12, %22 offset:0\n ds_read_b64_tr_b16 %13, %22 offset:4096\n"
            "ds_read_b64_tr_b16 %14, %23 offset:0\n ds_read_b64_tr_b16 %15, %23 offset:4096\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v0), "=&v"(w0), "=&v"(v1), "=&v"(w1), "=&v"(v2), "=&v"(w2), "=&v"(v3), "=&v"(w3),
              "=&v"(v4), "=&v"(w4), "=&v"(v5), "=&v"(w5), "=&v"(v6), "=&v"(w6), "=&v"(v7), "=&v"(w7)
            : "v"(sb + va[0]), "v"(sb + va[1]), "v"(sb + va[2]), "v"(sb + va[3]), "v"(sb + va[4]),
              "v"(sb + va[5]), "v"(sb + va[6]), "v"(sb + va[7])
            : "memory");
        const u32x2_t vlo[8] = {v0, v1, v2, v3, v4, v5, v6, v7};
        const u32x2_t vhi[8] = {w0, w1, w2, w3, w4, w5, w6, w7};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const u32x4_t vf = u32x4_t{vlo[dt].x, vlo[dt].y, vhi[dt].x, vhi[dt].y};
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh)
                o[hh][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, vf), __builtin_bit_cast(bf16x8_t, pf[hh]),
                    o[hh][dt], 0, 0, 0);
        }
    };

    // Tile 0 goes out first; iteration t waits for tile t (this wave's
    // loads, then every wave's at the barrier, after which tile t - 1's slot
    // is free), refills that slot with tile t + 1 and multiplies tile t.
    if (ntiles > 0) issue(0);
    f32x4_t sc[HPW][2];
    for (int t = 0; t < ntiles; ++t) {
        DG_WAIT_VM(0);
        attn_barrier();
        if (t + 1 < ntiles) issue(t + 1);
        const uint32_t sb = ring0 + (t % RING2) * SLOT2;
        qk(sb, sc);
        soft_pv(sb, kb + t * KT2, sc);
    }

    // lane holds O^T[d = dt*16 + 4*g4 + e][query r16]
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        float l_tot = l_run[hh] + __shfl_xor(l_run[hh], 16, 64);
        l_tot = l_tot + __shfl_xor(l_tot, 32, 64);
        if (!qvalid) continue;
        const int h = h0 + hh;
        if (a.splits == 1) {
            bf16_t* out = reinterpret_cast<bf16_t*>(a.out) + qrow * (long)a.Hq * DH + (long)h * DH;
            const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                uint2 w;
                w.x = pack_bf2(o[hh][dt][0] * inv, o[hh][dt][1] * inv);
                w.y = pack_bf2(o[hh][dt][2] * inv, o[hh][dt][3] * inv);
                *reinterpret_cast<uint2*>(out + dt * 16 + 4 * g4) = w;
            }
        } else {
            const long base = ((long)split * a.B * a.n + qrow) * a.Hq + h;
            float* po = a.part_o + base * DH;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                *reinterpret_cast<f32x4_t*>(po + dt * 16 + 4 * g4) = o[hh][dt];
            if (g4 == 0) {
                a.part_ml[base * 2 + 0] = m_run[hh];
                a.part_ml[base * 2 + 1] = l_tot;
            }
        }
    }
}

// ------------------------------------------------------------------------
// bf16, head dim 128, canvas (no mask but the key range): 32 queries of one
// query head per wave on the 32x32x16 MFMA, so every K and V fragment read
// from LDS serves twice the queries of attn2_kernel.
//   * S^T = K Q^T per 32-key tile: A = K (32 keys x 16 dh), B = Q^T; a lane
//     holds 16 keys (8(i/4) + 4g + i%4, g = lane/32) of query lane%32.
//   * The PV product takes the 32 keys as two halves of 16; with the
//     k-index of half h mapped to key 16h + 8(j/4) + 4g + j%4, lane l's B
//     operand is its own probabilities 8h..8h+7, and the A operand (V^T,
//     32 dh x 16 keys) is two transposing reads of 4 keys each.
//   * K rows: chunk c of row r in slot c ^ (r % 16); V rows: slot
//     c ^ 4(r % 4), so the 32 lanes of half a transposing read (4 rows x 4
//     chunks) touch 16 distinct slots, and rows 4 apart share a swizzle (the
//     second read of a fragment and the second key half are immediate
//     offsets).
constexpr int KT3 = 32;
constexpr int SLOT3 = 2 * TILE2;

__device__ __forceinline__ int swv3(int r) { return 4 * (r & 3); }

__global__ __launch_bounds__(256, 3) void attn3_kernel(AttnArgs a) {
    if (a.halt && *a.halt) return;
    constexpr int DH = 128;
    __shared__ __align__(1024) unsigned char ring[RING2 * SLOT3];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q32 = lane & 31, g = lane >> 5;
    const int G = a.Hq / a.Hkv;
    const int nqt = cdiv(a.n, 32);
    const int units = nqt * G;
    const int nx = cdiv(units, 4);
    const int ngroups = a.Hkv * a.B * a.splits;
    int bx, grp;
    if (ngroups % 8 == 0) {
        const int slot = blockIdx.x >> 3;
        bx = slot % nx;
        grp = (slot / nx) * 8 + (blockIdx.x & 7);
    } else {
        bx = blockIdx.x % nx;
        grp = blockIdx.x / nx;
    }
    const int kvh = grp % a.Hkv;
    const int b = (grp / a.Hkv) / a.splits, split = (grp / a.Hkv) % a.splits;
    const int unit = bx * 4 + wave;
    const bool wvalid = unit < units;
    const int qt = wvalid ? unit / G : 0;
    const int h = kvh * G + (wvalid ? unit % G : 0);
    const int qi = qt * 32 + q32;
    const bool qvalid = wvalid && qi < a.n;
    const long qrow = (long)b * a.n + (qvalid ? qi : 0);

    const int kb = split * a.split_len;
    const int ke = min(a.kv_len, kb + a.split_len);
    const int ntiles = ke > kb ? cdiv(ke - kb, KT3) : 0;

    // Q^T fragments (B operand): query q32, dh 16s + 8g .. +7, scaled so
    // that a score is log2-e based
    const float qscale = LOG2E / sqrtf((float)DH);
    u32x4_t qf[8];
    {
        const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.q) + qrow * (long)a.Hq * DH + (long)h * DH;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qvalid) v = *reinterpret_cast<const uint4*>(Q + 16 * s + 8 * g);
            qf[s] = u32x4_t{scale_bf2(v.x, qscale), scale_bf2(v.y, qscale), scale_bf2(v.z, qscale),
                            scale_bf2(v.w, qscale)};
        }
    }

    const bf16_t* Kc = reinterpret_cast<const bf16_t*>(a.kc) + ((long)b * a.Hkv + kvh) * (long)a.cap * DH;
    const bf16_t* Vc = reinterpret_cast<const bf16_t*>(a.vc) + ((long)b * a.Hkv + kvh) * (long)a.cap * DH;

    // direct-to-LDS fill: wave w writes 1 KiB blocks 2w and 2w+1 of each
    // tile; lane l of block q lands in row 4q + l/16, slot l%16
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int frow[2];
    uint32_t kof[2], vof[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        frow[i] = 4 * (2 * wv + i) + (lane >> 4);
        kof[i] = frow[i] * ROW2 + (((lane & 15) ^ (frow[i] & 15)) << 4);
        vof[i] = frow[i] * ROW2 + (((lane & 15) ^ swv3(frow[i])) << 4);
    }
    const char* Kb = reinterpret_cast<const char*>(Kc);
    const char* Vb = reinterpret_cast<const char*>(Vc);
    auto issue = [&](int t) {
        const int k0_ = kb + t * KT3;
        unsigned char* sl_ = ring + (t % RING2) * SLOT3 + 2 * wv * 1024;
        const char* kt_ = Kb + (long)k0_ * ROW2;
        const char* vt_ = Vb + (long)k0_ * ROW2;
        if (k0_ + KT3 <= ke) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                __builtin_amdgcn_global_load_lds((glb_void*)(kt_ + kof[i]), (lds_void*)(sl_ + i * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((glb_void*)(vt_ + vof[i]), (lds_void*)(sl_ + TILE2 + i * 1024), 16, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t r_ = min(frow[i], ke - 1 - k0_) * ROW2;
                __builtin_amdgcn_global_load_lds((glb_void*)(kt_ + r_ + (kof[i] & (ROW2 - 1))), (lds_void*)(sl_ + i * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((glb_void*)(vt_ + r_ + (vof[i] & (ROW2 - 1))), (lds_void*)(sl_ + TILE2 + i * 1024), 16, 0, 0);
            }
        }
    };

    // K fragment of dh slice s (A operand): row q32 (key), chunk 2s + g, in
    // slot (2s + g) ^ (q32 % 16): address ka0 ^ 32 s
    const uint32_t ring0 = lds_addr(ring);
    const uint32_t ka0 = q32 * ROW2 + ((g ^ (q32 & 1)) << 4) + (((q32 & 15) >> 1) << 5);
    // V^T fragment of dh block blk (A operand), first read of key half 0: the
    // 16-lane group q = lane/16 reads keys 4g + (lane%16)/4 (+0..3 after the
    // transpose), dh 32 blk + 16 (q % 2) + 4 (lane % 4) .. +3; the second read
    // is 8 keys on (+2048), key half 1 is 16 keys on (+4096)
    uint32_t va[4];
    {
        const int rv = 4 * g + ((lane & 15) >> 2);
        const int qh = (lane >> 4) & 1;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
            va[blk] = TILE2 + rv * ROW2 + (((4 * blk + 2 * qh + ((lane & 3) >> 1)) ^ swv3(rv)) << 4) +
                      8 * (lane & 1);
    }

    f32x16_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
    float m_run = -1e30f, l_run = 0.f;

    if (ntiles > 0) issue(0);
    for (int t = 0; t < ntiles; ++t) {
        DG_WAIT_VM(0);
        attn_barrier();
        if (t + 1 < ntiles) issue(t + 1);
        const uint32_t sb = ring0 + (t % RING2) * SLOT3;
        const int k0 = kb + t * KT3;

        // S^T - tile: two reads of four K slices each
        f32x16_t sc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            u32x4_t k0f, k1f, k2f, k3f;
            const uint32_t base = sb + ka0;
            asm volatile(
                "ds_read_b128 %0, %4\n ds_read_b128 %1, %5\n"
                "ds_read_b128 %2, %6\n ds_read_b128 %3, %7\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(k0f), "=&v"(k1f), "=&v"(k2f), "=&v"(k3f)
                : "v"(base ^ (uint32_t)(32 * (4 * part + 0))), "v"(base ^ (uint32_t)(32 * (4 * part + 1))),
                  "v"(base ^ (uint32_t)(32 * (4 * part + 2))), "v"(base ^ (uint32_t)(32 * (4 * part + 3)))
                : "memory");
            const u32x4_t kf[4] = {k0f, k1f, k2f, k3f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[s]),
                                                             __builtin_bit_cast(bf16x8_t, qf[4 * part + s]),
                                                             sc, 0, 0, 0);
        }

        // softmax of the lane's 16 keys against the running maximum
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = sc[i];
        if (k0 + KT3 > ke) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + 8 * (i >> 2) + 4 * g + (i & 3);
                if (key >= ke) x[i] = -INFINITY;
            }
        }
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
        if (__ballot(mx > m_run + RESCALE_T)) {
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mn = fmaxf(m_run, mx);
            const float corr = __builtin_amdgcn_exp2f(m_run - mn);
            l_run *= corr;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[blk][e] *= corr;
            m_run = mn;
        }
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_run);
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ls += p[i];
        l_run += ls;
        u32x4_t pf[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            pf[hh] = u32x4_t{pack_bf2(p[8 * hh + 0], p[8 * hh + 1]), pack_bf2(p[8 * hh + 2], p[8 * hh + 3]),
                             pack_bf2(p[8 * hh + 4], p[8 * hh + 5]), pack_bf2(p[8 * hh + 6], p[8 * hh + 7])};

        // O^T += V^T P^T: per pair of dh blocks, both key halves
#pragma unroll
        for (int bp = 0; bp < 2; ++bp) {
            u32x2_t a0, a1, a2, a3, b0, b1, b2, b3;
            asm volatile(
                "ds_read_b64_tr_b16 %0, %8 offset:0\n ds_read_b64_tr_b16 %1, %8 offset:2048\n"
                "ds_read_b64_tr_b16 %2, %8 offset:4096\n ds_read_b64_tr_b16 %3, %8 offset:6144\n"
                "ds_read_b64_tr_b16 %4, %9 offset:0\n ds_read_b64_tr_b16 %5, %9 offset:2048\n"
                "ds_read_b64_tr_b16 %6, %9 offset:4096\n ds_read_b64_tr_b16 %7, %9 offset:6144\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
                : "v"(sb + va[2 * bp]), "v"(sb + va[2 * bp + 1])
                : "memory");
            const u32x4_t v00 = u32x4_t{a0.x, a0.y, a1.x, a1.y}, v01 = u32x4_t{a2.x, a2.y, a3.x, a3.y};
            const u32x4_t v10 = u32x4_t{b0.x, b0.y, b1.x, b1.y}, v11 = u32x4_t{b2.x, b2.y, b3.x, b3.y};
            o[2 * bp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v00),
                                                                __builtin_bit_cast(bf16x8_t, pf[0]), o[2 * bp], 0, 0, 0);
            o[2 * bp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v01),
                                                                __builtin_bit_cast(bf16x8_t, pf[1]), o[2 * bp], 0, 0, 0);
            o[2 * bp + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v10),
                                                                    __builtin_bit_cast(bf16x8_t, pf[0]), o[2 * bp + 1], 0, 0, 0);
            o[2 * bp + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v11),
                                                                    __builtin_bit_cast(bf16x8_t, pf[1]), o[2 * bp + 1], 0, 0, 0);
        }
    }

    // lane holds O^T[dh = 32 blk + 8 (i/4) + 4 g + i%4][query q32]
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (!qvalid) return;
    if (a.splits == 1) {
        bf16_t* out = reinterpret_cast<bf16_t*>(a.out) + qrow * (long)a.Hq * DH + (long)h * DH;
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint2 w;
                w.x = pack_bf2(o[blk][4 * r + 0] * inv, o[blk][4 * r + 1] * inv);
                w.y = pack_bf2(o[blk][4 * r + 2] * inv, o[blk][4 * r + 3] * inv);
                *reinterpret_cast<uint2*>(out + 32 * blk + 8 * r + 4 * g) = w;
            }
    } else {
        const long base = ((long)split * a.B * a.n + qrow) * a.Hq + h;
        float* po = a.part_o + base * DH;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<f32x4_t*>(po + 32 * blk + 8 * r + 4 * g) =
                    f32x4_t{o[blk][4 * r + 0], o[blk][4 * r + 1], o[blk][4 * r + 2], o[blk][4 * r + 3]};
        if (g == 0) {
            a.part_ml[base * 2 + 0] = m_run;
            a.part_ml[base * 2 + 1] = l_tot;
        }
    }
}

// Merge of split partials: one workgroup of DH threads per (token, head).
template <typename T>
__global__ void attn_merge_kernel(AttnArgs a) {
    if (a.halt && *a.halt) return;
    const long th = blockIdx.x;            // token * Hq + head
    const int d = threadIdx.x;
    const long stride = (long)a.B * a.n * a.Hq;
    // the first wave reads every split's (max, sum) at once (splits <= 32)
    // and leaves the split weights and the total in LDS
    __shared__ float wts[32];
    __shared__ float ltot;
    if (d < 64) {
        const bool on = d < a.splits;
        const float ms = on ? a.part_ml[(d * stride + th) * 2] : -1e30f;
        const float ls = on ? a.part_ml[(d * stride + th) * 2 + 1] : 0.f;
        const float m = wave_max(ms);
        const float w = on ? exp2f(ms - m) : 0.f;
        const float l = wave_sum(w * ls);
        if (on) wts[d] = w;
        if (d == 0) ltot = l;
    }
    __syncthreads();
    float acc = 0.f;
    for (int s = 0; s < a.splits; ++s) acc += wts[s] * a.part_o[(s * stride + th) * a.dh + d];
    const float lsum = ltot;
    T* out = reinterpret_cast<T*>(a.out);
    out[th * a.dh + d] = Elt<T>::from_f(lsum > 0.f ? acc / lsum : 0.f);
}

}  // namespace

// bf16 with head dim 128 goes to attn3_kernel (canvas, no mask) or
// attn2_kernel (causal, one query head per wave).
bool attn2_takes(int dh, bool bf16) { return bf16 && dh == 128; }
int attn2_hpw(int) { return 1; }

int attention_splits(int B, int n, int Hq, int Hkv, int kv_len, int causal, int max_splits,
                     int* split_len, int dh, bool bf16) {
    const int G = Hq / Hkv;
    // workgroups of one key range, and the number to aim for: attn_kernel
    // runs eight small workgroups per CU, attn2_kernel four, attn3_kernel
    // three
    const bool v2 = attn2_takes(dh, bf16);
    const bool v3 = v2 && !causal;
    const long base = v3 ? (long)cdiv(cdiv(n, 32) * G, 4) * Hkv * B
                    : v2 ? (long)cdiv(cdiv(n, 16) * (G / attn2_hpw(G)), 4) * Hkv * B
                         : (long)cdiv(G * cdiv(n, 16), 4) * Hkv * B;
    const int target = v3 ? 768 : v2 ? 1024 : 2048;
    int splits = 1;
    if (!causal && kv_len > 256) {
        splits = (int)std::min<long>(cdiv(kv_len, 256), std::max<long>(1, cdiv(target, (int)base)));
        splits = std::min(splits, std::min(32, std::max(1, max_splits)));
    } else if (causal && n <= 16 && kv_len > 2 * KT) {
        // a decode step: a handful of queries over a long cache, so the
        // keys split into ranges of at least two tiles; a query's keys past
        // its position are masked in every range, and a range with no
        // visible key merges with weight 0
        splits = (int)std::min<long>(cdiv(kv_len, 2 * KT), std::max<long>(1, cdiv(target, (int)base)));
        splits = std::min(splits, std::min(32, std::max(1, max_splits)));
    }
    if (v2 && splits > 1) {
        // round to a count that makes (KV heads x sequences x splits) a
        // multiple of 8, so that attn2_kernel and attn3_kernel can keep each
        // key range on one XCD
        int g = Hkv * B, m = 8;
        while (m > 1 && g % 2 == 0) {
            g /= 2;
            m /= 2;
        }
        if (splits >= m) splits = (splits / m) * m;
    }
    int len = cdiv(cdiv(kv_len, splits), KT) * KT;
    if (len <= 0) len = KT;
    *split_len = len;
    return cdiv(std::max(kv_len, 1), len);
}

template <typename T>
hipError_t attention(const AttnArgs& a, hipStream_t st) {
    if (a.n <= 0 || a.B <= 0) return hipSuccess;
    // the merge keeps the split weights in one wave
    if (a.splits > 1 && (a.splits > 32 || a.dh < 64)) return hipErrorInvalidValue;
    const int G = a.Hq / a.Hkv;
    if (attn2_takes(a.dh, sizeof(T) == 2) && !a.causal) {
        dim3 grid3(cdiv(cdiv(a.n, 32) * G, 4) * a.Hkv * a.B * a.splits);
        hipLaunchKernelGGL(attn3_kernel, grid3, dim3(256), 0, st, a);
    } else if (attn2_takes(a.dh, sizeof(T) == 2)) {
        const int hpw = attn2_hpw(G);
        dim3 grid2(cdiv(cdiv(a.n, 16) * (G / hpw), 4) * a.Hkv * a.B * a.splits);
        hipLaunchKernelGGL(attn2_kernel<1>, grid2, dim3(256), 0, st, a);
    } else {
    dim3 grid(cdiv(G * cdiv(a.n, 16), 4), a.Hkv, a.B * a.splits);
    switch (a.dh) {
        case 64: hipLaunchKernelGGL((attn_kernel<T, 64>), grid, dim3(256), 0, st, a); break;
        case 128: hipLaunchKernelGGL((attn_kernel<T, 128>), grid, dim3(256), 0, st, a); break;
        case 256:
            if constexpr (sizeof(T) == 2) {
                hipLaunchKernelGGL((attn_kernel<T, 256>), grid, dim3(256), 0, st, a);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(attn_merge_kernel<T>, dim3((unsigned)((long)a.B * a.n * a.Hq)),
                       dim3(a.dh), 0, st, a);
    return hipGetLastError();
}

template hipError_t attention<bf16_t>(const AttnArgs&, hipStream_t);
template hipError_t attention<float>(const AttnArgs&, hipStream_t);

}  // namespace dg
