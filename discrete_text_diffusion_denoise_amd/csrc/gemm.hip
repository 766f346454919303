// Dense GEMMs of the denoising step on gfx950 MFMA.
//
//   C[M,N] (op)= A[M,K] * B[N,K]^T      (both operands K-contiguous)
//
// Used for the Q/K/V and output projections, the router, the self-
// conditioning projection, the tied logit head (report-summary page,
// sections 2 and 5: the denoiser reuses the autoregressive model's weights;
// sampling needs the full distribution of every canvas position) and the
// self-conditioning product softmax(L_prev) E (split over the vocabulary).
//
// Tiling: a workgroup owns a BM x BN tile and walks K in 128-byte slices
// (64 bf16 or 32 fp32), staging both operands in LDS with double buffering.
// Waves are arranged WM x WN; each wave owns (BM/WM) x (BN/WN) as 16x16
// MFMA tiles.  fp32 models use the same code with the 16x16x4 fp32 MFMA.
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace dg {

namespace {

constexpr int ROWB = 128;       // bytes of K per LDS row per slice
constexpr int PADB = 16;        // LDS row padding (bytes)
constexpr int LDSROW = ROWB + PADB;

template <typename T>
struct SliceTraits {
    static constexpr int BK = ROWB / (int)sizeof(T);          // K elements per slice
    static constexpr int KSTEPS = BK / 32;                     // MFMA k-steps per slice
    static constexpr int CE = 16 / (int)sizeof(T);            // elements per 16-byte chunk
    static constexpr int ROWE = LDSROW / (int)sizeof(T);      // LDS row stride (elements)
};

// --- operand loaders: 16-byte chunk (CE elements of T) at (row, k) -------

template <typename T, int AMODE>
struct ALoader;

// Plain row-major A (optionally gathered rows).
template <typename T>
struct ALoader<T, 0> {
    __device__ static uint4 load(const GemmArgs& g, int row, int k) {
        const T* A = reinterpret_cast<const T*>(g.A);
        long r = g.a_rows ? (long)g.a_rows[row] : (long)row;
        return *reinterpret_cast<const uint4*>(A + r * g.lda + k);
    }
};

// A = softmax(logits) row-wise, from fp32 logits and per-row {max, sum}.
template <>
struct ALoader<bf16_t, 1> {
    __device__ static uint4 load(const GemmArgs& g, int row, int k) {
        const float* L = reinterpret_cast<const float*>(g.A) + (long)row * g.lda + k;
        float m = g.a_stats[(long)row * 4 + 0];
        float inv = 1.0f / g.a_stats[(long)row * 4 + 1];
        float4 x0 = *reinterpret_cast<const float4*>(L);
        float4 x1 = *reinterpret_cast<const float4*>(L + 4);
        uint4 o;
        o.x = pack_bf2(__expf(x0.x - m) * inv, __expf(x0.y - m) * inv);
        o.y = pack_bf2(__expf(x0.z - m) * inv, __expf(x0.w - m) * inv);
        o.z = pack_bf2(__expf(x1.x - m) * inv, __expf(x1.y - m) * inv);
        o.w = pack_bf2(__expf(x1.z - m) * inv, __expf(x1.w - m) * inv);
        return o;
    }
};
template <>
struct ALoader<float, 1> {
    __device__ static uint4 load(const GemmArgs& g, int row, int k) {
        const float* L = reinterpret_cast<const float*>(g.A) + (long)row * g.lda + k;
        float m = g.a_stats[(long)row * 4 + 0];
        float inv = 1.0f / g.a_stats[(long)row * 4 + 1];
        float4 x = *reinterpret_cast<const float4*>(L);
        float4 p = make_float4(__expf(x.x - m) * inv, __expf(x.y - m) * inv,
                               __expf(x.z - m) * inv, __expf(x.w - m) * inv);
        return __builtin_bit_cast(uint4, p);
    }
};

template <typename T, int BM, int BN, int WM, int WN, int AMODE, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_tn_kernel(GemmArgs g) {
    using ST = SliceTraits<T>;
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM / 16;
    constexpr int TN = BN / WN / 16;
    constexpr int A_CHUNKS = BM * 8 / NT;   // 16-byte chunks per thread per slice
    constexpr int B_CHUNKS = BN * 8 / NT;
    static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for the thread count");

    extern __shared__ __align__(16) unsigned char smem[];
    T* As = reinterpret_cast<T*>(smem);                       // [2][BM][ROWE]
    T* Bs = As + 2 * BM * ST::ROWE;                            // [2][BN][ROWE]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int r16 = lane & 15, g4 = lane >> 4;

    // With xcd_group, the column tiles of one k-split are placed on one XCD
    // (workgroups are dealt to the 8 XCDs round-robin) so they share its L2.
    int nt = blockIdx.x, kz = blockIdx.z;
    if (g.xcd_group) {
        const int nx = gridDim.x;
        const int lin = blockIdx.x + nx * blockIdx.z;
        nt = (lin >> 3) % nx;
        kz = ((lin >> 3) / nx) * 8 + (lin & 7);
    }
    const int n0 = nt * BN;
    const int m0 = blockIdx.y * BM;
    const int kbeg = kz * g.k_split;
    const int kend = min(g.K, kbeg + g.k_split);
    const int nslices = cdiv(kend - kbeg, ST::BK);

    uint4 ra[A_CHUNKS], rb[B_CHUNKS];

    // Workgroups start their K walk at different slices (rotation by tile),
    // so concurrent workgroups read different offsets within their rows.
    const int rot = g.k_rotate && nslices > 0 ? (int)((nt + (long)blockIdx.y * 7) % nslices) : 0;
    auto gload = [&](int s) {
        int sr = s + rot;
        if (sr >= nslices) sr -= nslices;
        const int kb = kbeg + sr * ST::BK;
#pragma unroll
        for (int c = 0; c < A_CHUNKS; ++c) {
            int ch = tid + c * NT;
            int row = ch >> 3, kc = (ch & 7) * ST::CE;
            int gr = m0 + row, gk = kb + kc;
            if (gr < g.M && gk < kend)
                ra[c] = ALoader<T, AMODE>::load(g, gr, gk);
            else
                ra[c] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < B_CHUNKS; ++c) {
            int ch = tid + c * NT;
            int row = ch >> 3, kc = (ch & 7) * ST::CE;
            int gn = n0 + row, gk = kb + kc;
            if (gn < g.N && gk < kend) {
                if (sizeof(T) == 4 && g.b_bf16) {
                    // bf16 weights widened on load (exact)
                    const uint2 h = *reinterpret_cast<const uint2*>(b_row<bf16_t>(g, gn) + gk);
                    rb[c] = make_uint4(h.x << 16, h.x & 0xffff0000u, h.y << 16, h.y & 0xffff0000u);
                } else {
                    rb[c] = *reinterpret_cast<const uint4*>(b_row<T>(g, gn) + gk);
                }
            } else {
                rb[c] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto sstore = [&](int buf) {
        T* a = As + buf * BM * ST::ROWE;
        T* b = Bs + buf * BN * ST::ROWE;
#pragma unroll
        for (int c = 0; c < A_CHUNKS; ++c) {
            int ch = tid + c * NT;
            *reinterpret_cast<uint4*>(a + (ch >> 3) * ST::ROWE + (ch & 7) * ST::CE) = ra[c];
        }
#pragma unroll
        for (int c = 0; c < B_CHUNKS; ++c) {
            int ch = tid + c * NT;
            *reinterpret_cast<uint4*>(b + (ch >> 3) * ST::ROWE + (ch & 7) * ST::CE) = rb[c];
        }
    };

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (nslices > 0) {
        gload(0);
        sstore(0);
    }
    __syncthreads();

    const int arow0 = wm * (BM / WM) + r16;
    const int bcol0 = wn * (BN / WN) + r16;
    for (int s = 0; s < nslices; ++s) {
        const int buf = s & 1;
        if (s + 1 < nslices) gload(s + 1);
        const T* a = As + buf * BM * ST::ROWE;
        const T* b = Bs + buf * BN * ST::ROWE;
#pragma unroll
        for (int ks = 0; ks < ST::KSTEPS; ++ks) {
            Frag<T> fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                load_frag(fa[i], a + (arow0 + 16 * i) * ST::ROWE + ks * 32 + g4 * 8);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                load_frag(fb[j], b + (bcol0 + 16 * j) * ST::ROWE + ks * 32 + g4 * 8);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) mma(acc[i][j], fa[i], fb[j]);
        }
        if (s + 1 < nslices) sstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds rows 4*g4+e, column r16 of each 16x16 tile
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * (BN / WN) + 16 * j + r16;
            if (col >= g.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm * (BM / WM) + 16 * i + 4 * g4 + e;
                if (row >= g.M) continue;
                const float v = acc[i][j][e];
                if constexpr (EPI == EPI_STORE_F32) {
                    reinterpret_cast<float*>(g.C)[(long)row * g.ldc + col] = v;
                } else if constexpr (EPI == EPI_ADD_F32) {
                    reinterpret_cast<float*>(g.C)[(long)row * g.ldc + col] += v;
                } else if constexpr (EPI == EPI_SPLITK) {
                    reinterpret_cast<float*>(g.C)[((long)kz * g.M + row) * g.ldc + col] = v;
                } else if constexpr (EPI == EPI_EMBED_ADD) {
                    const T* E = reinterpret_cast<const T*>(g.E);
                    const long tok = min(max(g.tokens[row], 0), g.vocab - 1);
                    reinterpret_cast<float*>(g.C)[(long)row * g.ldc + col] =
                        v + Elt<T>::to_f(E[tok * g.lde + col]);
                }
            }
        }
    }
}

template <typename T, int BM, int BN, int WM, int WN, int AMODE, int EPI>
hipError_t launch_cfg(const GemmArgs& g, int splits, hipStream_t st) {
    using ST = SliceTraits<T>;
    dim3 grid(cdiv(g.N, BN), cdiv(g.M, BM), splits);
    size_t lds = (size_t)2 * (BM + BN) * ST::ROWE * sizeof(T);
    auto kern = gemm_tn_kernel<T, BM, BN, WM, WN, AMODE, EPI>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, grid, dim3(WM * WN * 64), lds, st, g);
    return hipGetLastError();
}

template <typename T, int AMODE, int EPI>
hipError_t launch_sized(const GemmArgs& g, int splits, hipStream_t st) {
    // Pick the largest tile that still gives the chip enough workgroups.
    long big = (long)cdiv(g.M, 256) * cdiv(g.N, 256) * splits;
    long med = (long)cdiv(g.M, 128) * cdiv(g.N, 128) * splits;
    // bf16 products with enough 256 x 256 tiles for every CU: the
    // direct-to-LDS ring kernel
    if constexpr (sizeof(T) == 2 && AMODE == 0 && (EPI == EPI_STORE_F32 || EPI == EPI_SPLITK)) {
        if (big >= 128 && gemm_dma_ok(g, EPI)) return gemm_dma_bf16(g, EPI, splits, st);
    }
    if (big >= 240) {
        // 256 x 256: eight waves of 128 x 64 (measured faster than four waves of
        // 128 x 128, which halve LDS reads but have half the loads in flight)
        return launch_cfg<T, 256, 256, 2, 4, AMODE, EPI>(g, splits, st);
    }
    if (med >= 200) return launch_cfg<T, 128, 128, 2, 2, AMODE, EPI>(g, splits, st);
    return launch_cfg<T, 64, 64, 2, 2, AMODE, EPI>(g, splits, st);
}

}  // namespace

template <typename T>
hipError_t gemm_tn(const GemmArgs& g, int amode, int epi, int splits, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    // blocked operands and slab maxima exist only for the bf16 ring kernel
    if (g.a_tiled || g.b_tiled || g.rowmax) {
        if (sizeof(T) != 2 || amode != 0) return hipErrorInvalidValue;
        return gemm_dma_bf16(g, epi, splits, st);
    }
    if (amode == 1) {
        if (epi != EPI_SPLITK) return hipErrorInvalidValue;
        return launch_sized<T, 1, EPI_SPLITK>(g, splits, st);
    }
    switch (epi) {
        case EPI_STORE_F32: return launch_sized<T, 0, EPI_STORE_F32>(g, splits, st);
        case EPI_ADD_F32: return launch_sized<T, 0, EPI_ADD_F32>(g, splits, st);
        case EPI_EMBED_ADD: return launch_sized<T, 0, EPI_EMBED_ADD>(g, splits, st);
        case EPI_SPLITK: return launch_sized<T, 0, EPI_SPLITK>(g, splits, st);
        default: return hipErrorInvalidValue;
    }
}

template hipError_t gemm_tn<bf16_t>(const GemmArgs&, int, int, int, hipStream_t);
template hipError_t gemm_tn<float>(const GemmArgs&, int, int, int, hipStream_t);

}  // namespace dg
