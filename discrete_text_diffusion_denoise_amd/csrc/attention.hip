// Grouped-query attention over the KV cache on gfx950 MFMA.
//
// The denoiser's canvas queries see every cached context key and every
// canvas key (no mask); the encoder's queries see keys up to their own
// position (causal).  Report-summary page (animattoys.com), section 2;
// youleyou.com article, "Architecture basis".
//
// A wave owns 16 queries of one query head; the four waves of a workgroup
// share one KV head, so each K/V tile staged in LDS serves all of them.
// Scores are computed transposed, S^T = K Q^T, so that a lane holds 8 keys of
// ONE query: the online-softmax state (max, sum, rescale) is lane-local
// except for one max across the 4 lanes of a query, and the probabilities
// already sit in the B-operand layout of O^T = V^T P^T.  Long key ranges are
// split across workgroups and merged by a second kernel.
#include <algorithm>
#include <cstdlib>

#include "common.h"
#include "kernels.h"

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

int attention_splits(int B, int n, int Hq, int Hkv, int kv_len, int causal, int max_splits,
                     int* split_len) {
    const int G = Hq / Hkv;
    const long base = (long)cdiv(G * cdiv(n, 16), 4) * Hkv * B;
    int splits = 1;
    // workgroups to aim for (eight per CU)
    constexpr int target = 2048;
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
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(attn_merge_kernel<T>, dim3((unsigned)((long)a.B * a.n * a.Hq)),
                       dim3(a.dh), 0, st, a);
    return hipGetLastError();
}

template hipError_t attention<bf16_t>(const AttnArgs&, hipStream_t);
template hipError_t attention<float>(const AttnArgs&, hipStream_t);

}  // namespace dg
