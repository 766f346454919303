// The tied head for decode steps of the retained autoregressive mode:
//
//   logits[M, V] = norm(h)[M, d] * E[V, d]^T,   M <= 16 new tokens
//
// (report-summary page, section 2: the output head is the tied embedding;
// sections 5 and 7: the same weights also decode as a causal language model,
// one new token per sequence per step).  The weight (1 GiB at V 262144, d 2048) dominates the step, and the
// vocabulary GEMM's 256-row output tile would spend its MFMA issue on padding
// rows, so this kernel keeps only the few rows of A and streams E:
//
//   * a 16 x 256 output tile per workgroup, four waves of 16 x 64;
//   * the 16 rows of A (both operands in the 256 x 32 blocked layout, K at
//     most 2048) copied once into LDS, each row padded by 16 bytes so the
//     fragment reads of 16 rows spread over the banks; rows past M are zero;
//   * E in 32-element k stages straight from global memory into a ring of
//     four 16 KiB LDS buffers (three in flight while one is multiplied), each
//     wave waiting only for its own oldest loads, the same swizzle of the
//     16-byte chunks as the vocabulary GEMM;
//   * optional 64-column slab maxima of each row in the epilogue (the greedy
//     choice reads them instead of the logits).
#include "common.h"
#include "kernels.h"
#include "lds_ring.h"

namespace dg {

namespace {

constexpr int BN = 256;
constexpr int BK = 32;                       // bf16 per row per stage (64 bytes)
constexpr int STAGE_BYTES = BN * BK * 2;     // one stage of the weight: 16 KiB
constexpr int DEC_KMAX = 2048;
constexpr int DEC_AST = DEC_KMAX * 2 + 16;   // LDS bytes per A row

__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs g) {
    if (g.halt && *g.halt) return;
    __shared__ __align__(1024) unsigned char b0[STAGE_BYTES], b1[STAGE_BYTES];
    __shared__ __align__(1024) unsigned char b2[STAGE_BYTES], b3[STAGE_BYTES];
    __shared__ __align__(16) unsigned char as[16 * DEC_AST];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int nt = blockIdx.x;
    const int n0 = nt * BN;
    const int n = __builtin_amdgcn_readfirstlane(g.K / BK);
    const int rot = __builtin_amdgcn_readfirstlane(g.k_rotate && n > 0 ? (int)(nt % n) : 0);

    // this wave fills blocks 4*wave .. 4*wave+3 of each stage (16 rows of
    // 64 bytes each; lane p writes slot p: row p/4, chunk (p%4) ^ swz(row))
    const bf16_t* B = reinterpret_cast<const bf16_t*>(g.B);
    const int pr = lane >> 2;
    const int pc = ((lane & 3) ^ swz(pr)) * 8;
    const bf16_t* pb = B + tiled_index(n0 + 64 * wave + pr, 0, g.K) + pc;
    const int blk0 = 4 * wave * 1024;

#define DD_ISSUE(s, SB)                                                                           \
    {                                                                                             \
        int sr_ = (s) + rot;                                                                      \
        if (sr_ >= n) sr_ -= n;                                                                   \
        const long kb_ = (long)sr_ * (256 * BK);                                                  \
        _Pragma("unroll") for (int q = 0; q < 4; ++q)                                             \
            __builtin_amdgcn_global_load_lds((glb_void*)(pb + kb_ + q * 16 * BK),                 \
                                             (lds_void*)((SB) + blk0 + q * 1024), 16, 0, 2);      \
    }
    if (n > 0) DD_ISSUE(0, b0);
    if (n > 1) DD_ISSUE(1, b1);
    if (n > 2) DD_ISSUE(2, b2);

    // A rows 0..15, all of K, into LDS (rows past M as zeros): stage s of the
    // blocked layout holds those rows' 32 values in its first 1 KiB
    const bf16_t* A = reinterpret_cast<const bf16_t*>(g.A);
    for (int c = tid; c < n * 64; c += 256) {
        const int s_ = c >> 6, e = (c & 63) * 8;
        const int row = e >> 5, kk = s_ * BK + (e & 31);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < g.M) v = *reinterpret_cast<const uint4*>(A + (long)s_ * (256 * BK) + e);
        *reinterpret_cast<uint4*>(as + row * DEC_AST + kk * 2) = v;
    }
    __syncthreads();

    f32x4_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int roff = r16 * 64 + ((g4 ^ swz(r16)) << 4);
    const uint32_t qa0 = lds_addr(as) + r16 * DEC_AST + g4 * 16;

#define DD_COMPUTE(SB, KS)                                                                        \
    {                                                                                             \
        u32x4 fa, e0, e1, e2, e3;                                                                 \
        int ks_ = (KS) + rot;                                                                     \
        if (ks_ >= n) ks_ -= n;                                                                   \
        const uint32_t qa_ = qa0 + ks_ * (BK * 2), qb_ = lds_addr(SB) + wave * 4096 + roff;       \
        asm volatile(                                                                             \
            "ds_read_b128 %0, %5\n"                                                               \
            "ds_read_b128 %1, %6 offset:0\n ds_read_b128 %2, %6 offset:1024\n"                     \
            "ds_read_b128 %3, %6 offset:2048\n ds_read_b128 %4, %6 offset:3072\n"                  \
            "s_waitcnt lgkmcnt(0)"                                                                 \
            : "=&v"(fa), "=&v"(e0), "=&v"(e1), "=&v"(e2), "=&v"(e3)                               \
            : "v"(qa_), "v"(qb_)                                                                  \
            : "memory");                                                                          \
        const u32x4 fb_[4] = {e0, e1, e2, e3};                                                    \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                             \
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                                     \
                __builtin_bit_cast(bf16x8_t, fb_[j]), __builtin_bit_cast(bf16x8_t, fa), acc[j],   \
                0, 0, 0);                                                                         \
    }
#define DD_STAGE(t, CB, NB)                  \
    {                                        \
        if ((t) + 2 < n)                     \
            DG_WAIT_VM(8);                   \
        else if ((t) + 1 < n)                \
            DG_WAIT_VM(4);                   \
        else                                 \
            DG_WAIT_VM(0);                   \
        barrier_lds();                       \
        if ((t) + 3 < n) DD_ISSUE((t) + 3, NB); \
        DD_COMPUTE(CB, t);                   \
    }
    for (int t = 0; t < n; t += 4) {
        DD_STAGE(t, b0, b3);
        DD_STAGE(t + 1, b1, b0);
        DD_STAGE(t + 2, b2, b1);
        DD_STAGE(t + 3, b3, b2);
    }
#undef DD_STAGE
#undef DD_COMPUTE
#undef DD_ISSUE

    // lane holds row r16, columns 16j + 4*g4 .. +3 of this wave's 64
    float* C = reinterpret_cast<float*>(g.C);
    const int row = r16;
    if (row < g.M) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wave * 64 + 16 * j + 4 * g4;
            *reinterpret_cast<f32x4_t*>(C + (long)row * g.ldc + col) = acc[j];
        }
    }
    if (g.rowmax) {
        float mx = acc[0][0];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) mx = max_nan(mx, acc[j][q]);
        mx = max_nan(mx, __shfl_xor(mx, 16, 64));
        mx = max_nan(mx, __shfl_xor(mx, 32, 64));
        const int nslab = g.N >> 6;
        if (g4 == 0 && row < g.M) g.rowmax[(long)row * nslab + nt * 4 + wave] = mx;
    }
}

}  // namespace

bool gemm_decode_ok(const GemmArgs& g) {
    return g.M >= 1 && g.M <= 16 && g.a_tiled == 1 && g.b_tiled == 1 && g.K <= DEC_KMAX &&
           g.K % (4 * BK) == 0 && g.N % BN == 0 && g.ldc % 4 == 0 && !g.a_rows &&
           (((uintptr_t)g.A | (uintptr_t)g.B | (uintptr_t)g.C) & 15) == 0;
}

hipError_t gemm_decode(const GemmArgs& g, hipStream_t st) {
    if (!gemm_decode_ok(g)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_decode_kernel, dim3(g.N / BN), dim3(256), 0, st, g);
    return hipGetLastError();
}

}  // namespace dg
