// Streaming bf16 GEMM for few rows and many columns:
//
//   C[M,N] (op)= A[M,K] * B[N,K]^T,  M <= 256 per row tile.
//
// This is the shape of the tied logit head (256 canvas positions x 262144
// vocabulary rows), of the self-conditioning product (256 positions x 2048
// over a 262144-long reduction) and of the per-layer projections at
// canvas size.  A workgroup owns all BM rows of a tile; the BM x 64 slice of
// A for each k-stage is staged once in LDS and shared by the 4 waves, while
// each wave streams its own 16*TN columns of B (embedding or weight rows)
// straight from HBM into MFMA registers, two stages ahead.  Every B element
// is therefore read from memory once and multiplied into all BM rows from
// registers; LDS carries only A (16 fragment reads per 16*TN MFMAs).
//
// Lane (g4, r16) of a 16x16x32 MFMA takes k = kb + g4*8*KS + s*8 + [0..7] for
// k-step s of a 32*KS-wide stage, in both operands, so each lane's B load is
// 16*KS contiguous bytes of one row.
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace dg {

namespace {

template <int TM, int TN, int KS, int WM, int EPI>
__global__ __launch_bounds__(256 * WM) void gemm_stream_kernel(GemmArgs g) {
    constexpr int NT = 256 * WM;        // threads: 4 column groups x WM row groups of waves
    constexpr int SKB = 32 * KS;        // k per stage (KS MFMA k-steps)
    constexpr int SROW = SKB + 8;       // LDS row stride (elements), 16-byte padded
    constexpr int CPR = SKB / 8;        // 16-byte chunks per A row per stage
    constexpr int BM = 16 * TM * WM;
    constexpr int WC = 16 * TN;
    constexpr int BN = 4 * WC;
    constexpr int ACH = BM * CPR / NT;  // 16-byte A chunks per thread per stage
    static_assert(ACH >= 1, "row tile too small");
    __shared__ __align__(16) bf16_t As[2][BM * SROW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int wn = wave & 3, wrow = (wave >> 2) * 16 * TM;   // column group, first row

    // Tile coordinates.  With xcd_group, the column tiles of one k-split are
    // placed on one XCD (workgroups are dealt to the 8 XCDs round-robin), so
    // they share that XCD's L2 for the A slices.
    int nt = blockIdx.x, mt = blockIdx.y, kz = blockIdx.z;
    if (g.xcd_group) {
        const int nx = gridDim.x;
        const int lin = blockIdx.x + nx * blockIdx.z;
        const int xcd = lin & 7, local = lin >> 3;
        nt = local % nx;
        kz = (local / nx) * 8 + xcd;
    }
    const int n0 = nt * BN + wn * WC;
    const int m0 = mt * BM;
    const int kbeg = kz * g.k_split;
    const int kend = min(g.K, kbeg + g.k_split);
    const int nst = kend > kbeg ? cdiv(kend - kbeg, SKB) : 0;
    const bf16_t* A = reinterpret_cast<const bf16_t*>(g.A);

    const bf16_t* brow[TN];
    bool bval[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = n0 + 16 * j + r16;
        bval[j] = col < g.N;
        brow[j] = b_row<bf16_t>(g, bval[j] ? col : 0);
    }

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

// A slice of stage ST -> registers ra
#define DG_ALOAD(ST)                                                                          \
    {                                                                                         \
        const int kb_ = kbeg + (ST) * SKB;                                                    \
        _Pragma("unroll") for (int c = 0; c < ACH; ++c) {                                     \
            const int ch = tid + c * NT;                                                      \
            const int gr = m0 + ch / CPR, gk = kb_ + (ch % CPR) * 8;                          \
            ra[c] = (gr < g.M && gk < kend)                                                   \
                        ? *reinterpret_cast<const uint4*>(A + (long)gr * g.lda + gk)          \
                        : make_uint4(0, 0, 0, 0);                                             \
        }                                                                                     \
    }
// registers ra -> LDS buffer BUF
#define DG_ASTORE(BUF)                                                                        \
    {                                                                                         \
        _Pragma("unroll") for (int c = 0; c < ACH; ++c) {                                     \
            const int ch = tid + c * NT;                                                      \
            *reinterpret_cast<uint4*>(&As[BUF][(ch / CPR) * SROW + (ch % CPR) * 8]) = ra[c];  \
        }                                                                                     \
    }
// B columns of stage ST -> register set BS
#define DG_BLOAD(ST, BS)                                                                      \
    {                                                                                         \
        const int k_ = kbeg + (ST) * SKB + g4 * 8 * KS;                                       \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                      \
            _Pragma("unroll") for (int s_ = 0; s_ < KS; ++s_) {                               \
                BS[s_ * TN + j] = (bval[j] && k_ < kend)                                      \
                    ? *reinterpret_cast<const uint4*>(brow[j] + k_ + 8 * s_)                  \
                    : make_uint4(0, 0, 0, 0);                                                 \
            }                                                                                 \
        }                                                                                     \
    }
// MFMAs of one stage: A from LDS buffer BUF, B from register set BS
#define DG_COMPUTE(BUF, BS)                                                                   \
    _Pragma("unroll") for (int s_ = 0; s_ < KS; ++s_) {                                       \
        Frag<bf16_t> fb[TN];                                                                  \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[j].v = BS[s_ * TN + j];             \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) {                                      \
            Frag<bf16_t> fa;                                                                  \
            fa.v = *reinterpret_cast<const uint4*>(                                           \
                &As[BUF][(wrow + 16 * i + r16) * SROW + g4 * 8 * KS + s_ * 8]);               \
            _Pragma("unroll") for (int j = 0; j < TN; ++j) mma(acc[i][j], fa, fb[j]);         \
        }                                                                                     \
    }

    uint4 ra[ACH];
    uint4 bA[KS * TN], bB[KS * TN];   // two stages of B in flight
    if (nst > 0) {
        DG_ALOAD(0)
        DG_ASTORE(0)
        DG_BLOAD(0, bA)
        if (nst > 1) DG_BLOAD(1, bB)
    }
    __syncthreads();
    // stages in pairs so the two B register sets keep fixed names
    for (int st = 0; st < nst; st += 2) {
        if (st + 1 < nst) DG_ALOAD(st + 1)
        DG_COMPUTE(0, bA)
        if (st + 2 < nst) DG_BLOAD(st + 2, bA)
        if (st + 1 < nst) DG_ASTORE(1)
        __syncthreads();
        if (st + 1 >= nst) break;
        if (st + 2 < nst) DG_ALOAD(st + 2)
        DG_COMPUTE(1, bB)
        if (st + 3 < nst) DG_BLOAD(st + 3, bB)
        if (st + 2 < nst) DG_ASTORE(0)
        __syncthreads();
    }
#undef DG_ALOAD
#undef DG_ASTORE
#undef DG_BLOAD
#undef DG_COMPUTE

    // lane holds rows 4*g4 + e, column r16 of each 16x16 tile
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + 16 * j + r16;
            if (col >= g.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wrow + 16 * i + 4 * g4 + e;
                if (row >= g.M) continue;
                const float v = acc[i][j][e];
                if constexpr (EPI == EPI_STORE_F32) {
                    reinterpret_cast<float*>(g.C)[(long)row * g.ldc + col] = v;
                } else if constexpr (EPI == EPI_ADD_F32) {
                    reinterpret_cast<float*>(g.C)[(long)row * g.ldc + col] += v;
                } else if constexpr (EPI == EPI_SPLITK) {
                    reinterpret_cast<float*>(g.C)[((long)kz * g.M + row) * g.ldc + col] = v;
                } else if constexpr (EPI == EPI_EMBED_ADD) {
                    const bf16_t* E = reinterpret_cast<const bf16_t*>(g.E);
                    const long tok = min(max(g.tokens[row], 0), g.vocab - 1);
                    reinterpret_cast<float*>(g.C)[(long)row * g.ldc + col] =
                        v + bf2f(E[tok * g.lde + col]);
                }
            }
        }
    }
}

template <int TMW, int TN, int KS, int WM, int EPI>
hipError_t launch_cfg(const GemmArgs& g, int splits, hipStream_t st) {
    constexpr int BN = 4 * 16 * TN, BM = 16 * TMW * WM;
    dim3 grid(cdiv(g.N, BN), cdiv(g.M, BM), splits);
    hipLaunchKernelGGL((gemm_stream_kernel<TMW, TN, KS, WM, EPI>), grid, dim3(256 * WM), 0, st, g);
    return hipGetLastError();
}

template <int TM, int TN, int EPI>
hipError_t launch(const GemmArgs& g, int splits, hipStream_t st) {
    if constexpr (TM == 16 && TN == 4) {
        // wide tile of 256-row, many-column products: 256 x 256, 8 waves
        return launch_cfg<8, 4, 2, 2, EPI>(g, splits, st);
    } else {
        return launch_cfg<TM, TN, 2, 1, EPI>(g, splits, st);
    }
}

template <int EPI>
hipError_t launch_tiles(const GemmArgs& g, int tm, int tn, int splits, hipStream_t st) {
    if (tn == 4) {
        if (tm == 16) return launch<16, 4, EPI>(g, splits, st);
        if (tm == 8) return launch<8, 4, EPI>(g, splits, st);
        return launch<4, 4, EPI>(g, splits, st);
    }
    if (tm == 16) return launch<16, 1, EPI>(g, splits, st);
    if (tm == 8) return launch<8, 1, EPI>(g, splits, st);
    return launch<4, 1, EPI>(g, splits, st);
}

// (out, partials, splits, M, N, ldc) -> out[m][n] op= sum_z part[z][m][n]
__global__ __launch_bounds__(256) void splitk_epilogue_kernel(GemmArgs g, const float* part,
                                                              int splits, int epi) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const long total = (long)g.M * g.N;
    if (idx >= total) return;
    const int row = (int)(idx / g.N), col = (int)(idx % g.N);
    // the partials are summed in split order
    const float v = splitk_sum(part + (long)row * g.N + col, (long)g.M * g.N, splits);
    float* C = reinterpret_cast<float*>(g.C) + (long)row * g.ldc + col;
    if (epi == EPI_STORE_F32) {
        *C = v;
    } else if (epi == EPI_ADD_F32) {
        *C += v;
    } else {
        const long tok = min(max(g.tokens[row], 0), g.vocab - 1);
        if (g.E_is_f32)
            *C = v + reinterpret_cast<const float*>(g.E)[tok * g.lde + col];
        else
            *C = v + bf2f(reinterpret_cast<const bf16_t*>(g.E)[tok * g.lde + col]);
    }
}

}  // namespace

int stream_tm_for(int M) { return M <= 64 ? 4 : (M <= 128 ? 8 : 16); }

hipError_t gemm_stream(const GemmArgs& g, int epi, int tn, int splits, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    if (g.K % 16 != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0) return hipErrorInvalidValue;
    if (g.a_tiled || g.b_tiled || g.rowmax) return hipErrorInvalidValue;
    const int tm = stream_tm_for(g.M);
    switch (epi) {
        case EPI_STORE_F32: return launch_tiles<EPI_STORE_F32>(g, tm, tn, splits, st);
        case EPI_ADD_F32: return launch_tiles<EPI_ADD_F32>(g, tm, tn, splits, st);
        case EPI_SPLITK: return launch_tiles<EPI_SPLITK>(g, tm, tn, splits, st);
        case EPI_EMBED_ADD: return launch_tiles<EPI_EMBED_ADD>(g, tm, tn, splits, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t splitk_epilogue(const GemmArgs& g, const float* part, int splits, int epi,
                           hipStream_t st) {
    const long total = (long)g.M * g.N;
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(splitk_epilogue_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, st, g, part, splits, epi);
    return hipGetLastError();
}

}  // namespace dg
