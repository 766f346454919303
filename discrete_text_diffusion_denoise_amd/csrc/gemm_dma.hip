// The two vocabulary-sized bf16 GEMMs of the denoising step on gfx950:
//
//   logits[T, V]        = norm(h)[T, d] * E[V, d]^T        (tied head)
//   part_z[T, d]        = softmax(L_prev)[T, Vz] * E^T[d, Vz]^T   (self-
//                          conditioning, one vocabulary range Vz per k-split)
//
// (report-summary page, sections 2 and 5: the denoiser reuses the
// autoregressive model's tied embedding; self-conditioning feeds the previous
// step's distribution back through it.)  Both stream a 1 GiB weight once per
// call while the other operand (256 canvas rows) stays in L2, so the kernel
// is built around keeping many bytes of the streamed operand in flight:
//
//   * a 256 x 256 output tile per workgroup, eight waves of 128 x 64;
//   * K walked in 32-element stages (64 bytes per row) that go straight from
//     global memory into LDS with global_load_lds (no register staging);
//   * a ring of four stage slots per operand, three stages in flight while
//     the fourth is multiplied; each wave waits only for its own oldest
//     loads (vmcnt) and the barrier orders the LDS reads;
//   * an XOR swizzle of the 16-byte chunks inside every 64-byte row so that
//     the fragment reads (16 rows x one chunk per lane group) run at the LDS
//     rate of a linear read, chosen by which global chunk each lane fetches;
//   * for the head, a persistent grid (one workgroup per CU walking its
//     column tiles with one ring across tile boundaries, the row tiles of a
//     column tile on one XCD so that its L2 serves E to all of them).
//
// Rows past M or N are clamped to the last valid row (their results are
// never stored), so every load stays inside the operands.
#include <algorithm>
#include <cstdlib>

#include "common.h"
#include "kernels.h"
#include "lds_ring.h"

namespace dg {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;                 // bf16 per row per stage (64 bytes)
constexpr int WAVES = 8;               // arranged 2 (rows) x 4 (columns)
constexpr int STAGE_BYTES = BM * BK * 2;   // one operand's stage: 16 KiB

// vmcnt(m) for the largest even m <= c, m <= 12 (c is wave-uniform): waits
// until at most c of this wave's vector-memory operations are outstanding
__device__ __forceinline__ void wait_vm_upto(int c) {
    if (c >= 12)
        DG_WAIT_VM(12);
    else if (c >= 10)
        DG_WAIT_VM(10);
    else if (c >= 8)
        DG_WAIT_VM(8);
    else if (c >= 6)
        DG_WAIT_VM(6);
    else if (c >= 4)
        DG_WAIT_VM(4);
    else if (c >= 2)
        DG_WAIT_VM(2);
    else
        DG_WAIT_VM(0);
}

// One stage of a wave's 128 x 64 tile: eight 16-row A fragments at qa,
// qa + 1024, ..., four 16-row B fragments at qb, ..., 32 MFMAs.  The twelve
// fragment reads are one asm block that ends with its own lgkmcnt(0):
// written as ordinary loads, the compiler cannot tell at the top of the loop
// which ring slot a pending direct-to-LDS load targets and drains all of
// them (vmcnt(0)) once per pass.  The ring discipline already orders every
// read after the loads it needs.  Operands enter the MFMA swapped (B rows as
// the 16-row side), so a lane ends up holding four consecutive columns of
// one output row.
__device__ __forceinline__ void ring_mma(f32x4_t (&acc)[8][4], uint32_t qa, uint32_t qb) {
    u32x4 f0, f1, f2, f3, f4, f5, f6, f7, e0, e1, e2, e3;
    asm volatile(
        "ds_read_b128 %0, %12 offset:0\n ds_read_b128 %1, %12 offset:1024\n"
        "ds_read_b128 %2, %12 offset:2048\n ds_read_b128 %3, %12 offset:3072\n"
        "ds_read_b128 %4, %12 offset:4096\n ds_read_b128 %5, %12 offset:5120\n"
        "ds_read_b128 %6, %12 offset:6144\n ds_read_b128 %7, %12 offset:7168\n"
        "ds_read_b128 %8, %13 offset:0\n ds_read_b128 %9, %13 offset:1024\n"
        "ds_read_b128 %10, %13 offset:2048\n ds_read_b128 %11, %13 offset:3072\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f0), "=&v"(f1), "=&v"(f2), "=&v"(f3), "=&v"(f4), "=&v"(f5), "=&v"(f6), "=&v"(f7),
          "=&v"(e0), "=&v"(e1), "=&v"(e2), "=&v"(e3)
        : "v"(qa), "v"(qb)
        : "memory");
    const u32x4 fa[8] = {f0, f1, f2, f3, f4, f5, f6, f7};
    const u32x4 fb[4] = {e0, e1, e2, e3};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, fb[j]), __builtin_bit_cast(bf16x8_t, fa[i]), acc[i][j],
                0, 0, 0);
}

// BPOL: cache-policy bits of the B operand's loads (2 = non-temporal).
// D: ring slots per operand; stage s is loaded D - 1 stages ahead of its use.
// (One depth for both: a wave's loads complete in issue order, so waiting
// for one operand's stage also waits for every load of the other issued
// before it, and a deeper ring for one operand alone would hide no more
// latency.)
template <int EPI, int TA, int TB, int BPOL, int D>
__global__ __launch_bounds__(WAVES * 64) void gemm_dma_kernel(GemmArgs g) {
    static_assert(D >= 2 && 2 * D * STAGE_BYTES <= 160 * 1024, "ring");
    constexpr int P = D - 1;
    if (g.halt && *g.halt) return;
    __shared__ __align__(1024) unsigned char ra[D * STAGE_BYTES];
    __shared__ __align__(1024) unsigned char rb[D * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int r16 = lane & 15, g4 = lane >> 4;

    int nt = blockIdx.x, kz = blockIdx.z;
    if (g.xcd_group) {
        // the column tiles of one k-split land on one XCD and share its L2
        const int nx = gridDim.x;
        const int lin = blockIdx.x + nx * blockIdx.z;
        nt = (lin >> 3) % nx;
        kz = ((lin >> 3) / nx) * 8 + (lin & 7);
    }
    const int n0 = nt * BN;
    const int m0 = blockIdx.y * BM;
    const int kbeg = kz * g.k_split;
    const int kend = min(g.K, kbeg + g.k_split);
    // n and rot are the same in every lane; saying so keeps the stage
    // branches scalar
    const int n = __builtin_amdgcn_readfirstlane(kend > kbeg ? (kend - kbeg) / BK : 0);
    const int rot = __builtin_amdgcn_readfirstlane(g.k_rotate && n > 0 ? (int)((nt + blockIdx.y * 7) % n) : 0);

    // This wave fills blocks 2*wave and 2*wave+1 of both operands; lane p
    // writes LDS slot p of a block: row p/4, slot p%4, which holds chunk
    // (p%4) ^ swz(row).
    const bf16_t* A = reinterpret_cast<const bf16_t*>(g.A);
    const bf16_t* B = reinterpret_cast<const bf16_t*>(g.B);
    const int pr = lane >> 2;
    const int pc = ((lane & 3) ^ swz(pr)) * 8;
    // row-major: rows clamped to the last valid row; tiled: the padded
    // rows exist, and a stage of a 256-row tile is one 16 KiB block
    const bf16_t *pa0, *pa1, *pb0, *pb1;
    if (TA == 1) {
        pa0 = A + tiled_index(m0 + 32 * wave + pr, kbeg, g.K) + pc;
        pa1 = pa0 + 16 * 32;
    } else if (TA == 2) {
        pa0 = A + tiled64_index(m0 + 32 * wave + pr, kbeg, g.K) + pc;
        pa1 = pa0 + 16 * 64;
    } else {
        const long ar0 = min(m0 + 32 * wave + pr, g.M - 1), ar1 = min(m0 + 32 * wave + 16 + pr, g.M - 1);
        pa0 = A + ar0 * g.lda + kbeg + pc;
        pa1 = A + ar1 * g.lda + kbeg + pc;
    }
    if (TB) {
        pb0 = B + tiled_index(n0 + 32 * wave + pr, kbeg, g.K) + pc;
        pb1 = pb0 + 16 * 32;
    } else {
        const long br0 = min(n0 + 32 * wave + pr, g.N - 1), br1 = min(n0 + 32 * wave + 16 + pr, g.N - 1);
        pb0 = B + br0 * g.ldb + kbeg + pc;
        pb1 = B + br1 * g.ldb + kbeg + pc;
    }
    constexpr int SA_STRIDE = TA ? 256 * BK : BK;      // elements from one stage to the next
    constexpr int SB_STRIDE = TB ? 256 * BK : BK;
    const int blk0 = 2 * wave * 1024;

    // stage s of either operand into ring slot s % D (two loads of each per
    // wave)
#define DG_ISSUE_A(s)                                                                             \
    {                                                                                             \
        int sr_ = (s) + rot;                                                                      \
        if (sr_ >= n) sr_ -= n;                                                                   \
        const long ka_ = TA == 2 ? (long)(sr_ >> 1) * (256 * 64) + (sr_ & 1) * 32                 \
                                 : (long)sr_ * SA_STRIDE;                                         \
        unsigned char* d_ = ra + ((s) % D) * STAGE_BYTES + blk0;                                  \
        __builtin_amdgcn_global_load_lds((glb_void*)(pa0 + ka_), (lds_void*)d_, 16, 0, 0);        \
        __builtin_amdgcn_global_load_lds((glb_void*)(pa1 + ka_), (lds_void*)(d_ + 1024), 16, 0, 0); \
    }
#define DG_ISSUE_B(s)                                                                             \
    {                                                                                             \
        int sr_ = (s) + rot;                                                                      \
        if (sr_ >= n) sr_ -= n;                                                                   \
        const long kb_ = (long)sr_ * SB_STRIDE;                                                   \
        unsigned char* d_ = rb + ((s) % D) * STAGE_BYTES + blk0;                                  \
        __builtin_amdgcn_global_load_lds((glb_void*)(pb0 + kb_), (lds_void*)d_, 16, 0, BPOL);     \
        __builtin_amdgcn_global_load_lds((glb_void*)(pb1 + kb_), (lds_void*)(d_ + 1024), 16, 0, BPOL); \
    }

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int roff = r16 * 64 + ((g4 ^ swz(r16)) << 4);
#define DG_COMPUTE(SA, SB) ring_mma(acc, lds_addr(SA) + wm * 8192 + roff, lds_addr(SB) + wn * 4096 + roff)

    // Stages 0 .. D - 2 go out before the loop; pass t waits for stage t
    // (the loads of the D - 2 later stages already issued may stay
    // outstanding: four per wave per stage), lets every wave pass the
    // barrier (stage t has landed everywhere, stage t - 1's slots are free),
    // refills those slots with stage t + D - 1 and multiplies.
    for (int j = 0; j < P; ++j)
        if (j < n) {
            DG_ISSUE_B(j);
            DG_ISSUE_A(j);
        }
    for (int t = 0; t < n; ++t) {
        wait_vm_upto(4 * (min(n - 1, t + P - 1) - t));
        barrier_lds();
        if (t + P < n) {
            DG_ISSUE_B(t + P);
            DG_ISSUE_A(t + P);
        }
        DG_COMPUTE(ra + (t % D) * STAGE_BYTES, rb + (t % D) * STAGE_BYTES);
    }
#undef DG_COMPUTE
#undef DG_ISSUE_A
#undef DG_ISSUE_B

    // epilogue: lane holds row r16, columns 4*g4 .. 4*g4+3 of each 16x16 tile
    float* C = reinterpret_cast<float*>(g.C) + (EPI == EPI_SPLITK ? (long)kz * g.M * g.ldc : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + wm * 128 + 16 * i + r16;
        if (row >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + 16 * j + 4 * g4;
            if (col < g.N) *reinterpret_cast<f32x4_t*>(C + (long)row * g.ldc + col) = acc[i][j];
        }
    }
    if (EPI == EPI_STORE_F32 && g.rowmax) {
        // maximum of each row over this wave's 64 columns: the four columns
        // of each of the four 16-column tiles in the lane, then the four
        // lanes (g4) that hold the same row
        const int nslab = g.N >> 6, slab = nt * 4 + wn;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float mx = acc[i][0][0];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) mx = max_nan(mx, acc[i][j][q]);
            mx = max_nan(mx, __shfl_xor(mx, 16, 64));
            mx = max_nan(mx, __shfl_xor(mx, 32, 64));
            const int row = m0 + wm * 128 + 16 * i + r16;
            if (g4 == 0 && row < g.M && slab < nslab) g.rowmax[(long)row * nslab + slab] = mx;
        }
    }
}

// Persistent form of the tied head (both operands blocked, fp32 logits,
// optional slab maxima, N a multiple of 256): about one workgroup per CU,
// each walking a sequence of column tiles of one row tile with one ring
// across the tile boundaries.  The first stages of the next tile are in
// flight while a finished tile's logits are written; with one tile per
// workgroup every CU would drain its ring, write 256 KiB and refill it at
// the same moment, four times per call.
//
// Workgroups go to the eight XCDs in turn (w -> XCD w % 8).  On each XCD the
// G = rtiles row tiles of a column tile run side by side, walking its k
// stages in the same order, so the XCD's L2 serves E to G workgroups for one
// read from HBM; there are 8 * CG such column lanes (CG = slots per XCD / G),
// lane c taking column tiles c, c + 8 CG, ...
template <int D>
__global__ __launch_bounds__(WAVES * 64) void gemm_head_kernel(GemmArgs g, int rtiles) {
    constexpr int P = D - 1;
    if (g.halt && *g.halt) return;
    __shared__ __align__(1024) unsigned char ra[D * STAGE_BYTES];
    __shared__ __align__(1024) unsigned char rb[D * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int w = blockIdx.x;
    const int slots = gridDim.x / 8;                  // workgroups per XCD
    const int CG = slots / rtiles;                    // column lanes per XCD
    const int s_ = w / 8;
    if (s_ >= CG * rtiles) return;                    // spare slot
    const int mt = s_ % rtiles;
    const int c0 = (w % 8) * CG + s_ / rtiles;        // this workgroup's column lane
    const int nlanes = 8 * CG;
    const int m0 = mt * BM;
    const int ntiles = g.N / BN;
    const int n = __builtin_amdgcn_readfirstlane(g.K / BK);   // stages per tile
    const int mine = __builtin_amdgcn_readfirstlane(c0 < ntiles ? (ntiles - 1 - c0) / nlanes + 1 : 0);
    const int U = mine * n;                                   // stages of this workgroup

    // this wave fills blocks 2*wave and 2*wave+1 of both operands' slots
    // (lane p: row p/4, chunk (p%4) ^ swz(row)); column tile nt of E starts
    // nt * 256 * K elements further
    const int pr = lane >> 2;
    const int pc = ((lane & 3) ^ swz(pr)) * 8;
    const bf16_t* pa = reinterpret_cast<const bf16_t*>(g.A) + tiled_index(m0 + 32 * wave + pr, 0, g.K) + pc;
    const bf16_t* pb = reinterpret_cast<const bf16_t*>(g.B) + tiled_index(32 * wave + pr, 0, g.K) + pc;
    const long tile_b = 256L * g.K;
    const int blk0 = 2 * wave * 1024;

    // issue cursor: column tile i_nt, stage i_k, k rotation of that tile
    // (the same for every row tile of a column tile)
    int i_nt = c0, i_k = 0;
    int i_rot = g.k_rotate ? i_nt % n : 0;
    auto issue = [&](int slot) {
        int sr = i_k + i_rot;
        if (sr >= n) sr -= n;
        const bf16_t* b_ = pb + i_nt * tile_b + (long)sr * (256 * BK);
        const bf16_t* a_ = pa + (long)sr * (256 * BK);
        unsigned char* db = rb + slot * STAGE_BYTES + blk0;
        unsigned char* da = ra + slot * STAGE_BYTES + blk0;
        __builtin_amdgcn_global_load_lds((glb_void*)b_, (lds_void*)db, 16, 0, 2);
        __builtin_amdgcn_global_load_lds((glb_void*)(b_ + 16 * BK), (lds_void*)(db + 1024), 16, 0, 2);
        __builtin_amdgcn_global_load_lds((glb_void*)a_, (lds_void*)da, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void*)(a_ + 16 * BK), (lds_void*)(da + 1024), 16, 0, 0);
        if (++i_k == n) {
            i_k = 0;
            i_nt += nlanes;
            i_rot = g.k_rotate ? i_nt % n : 0;
        }
    };

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int roff = r16 * 64 + ((g4 ^ swz(r16)) << 4);
    float* C = reinterpret_cast<float*>(g.C);
    const int nslab = g.N >> 6;

    for (int j = 0; j < P && j < U; ++j) issue(j);
    int c_nt = c0, c_k = 0;
    // the epilogue of a finished tile, after the pass that multiplied its
    // last stage
    auto tile_end = [&]() {
        if (++c_k < n) return;
        // tile c_nt done: lane holds row r16, columns 4*g4 .. 4*g4+3 of each
        // 16x16 block
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = m0 + wm * 128 + 16 * i + r16;
            if (row < g.M) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = c_nt * BN + wn * 64 + 16 * j + 4 * g4;
                    *reinterpret_cast<f32x4_t*>(C + (long)row * g.ldc + col) = acc[i][j];
                }
            }
            if (g.rowmax) {
                // the row's maximum over this wave's 64 columns
                float mx = acc[i][0][0];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) mx = max_nan(mx, acc[i][j][q]);
                mx = max_nan(mx, __shfl_xor(mx, 16, 64));
                mx = max_nan(mx, __shfl_xor(mx, 32, 64));
                if (g4 == 0 && row < g.M) g.rowmax[(long)row * nslab + c_nt * 4 + wn] = mx;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        c_k = 0;
        c_nt += nlanes;
    };
    for (int u = 0; u < U; ++u) {
        // stage u has landed once at most the loads of the stages issued
        // after it are outstanding (four per wave and stage; loads complete
        // in issue order; the logits stores of a finished tile only make this
        // wait longer)
        wait_vm_upto(4 * (min(U - 1, u + P - 1) - u));
        barrier_lds();
        if (u + P < U) issue((u + P) % D);
        ring_mma(acc, lds_addr(ra + (u % D) * STAGE_BYTES) + wm * 8192 + roff,
                 lds_addr(rb + (u % D) * STAGE_BYTES) + wn * 4096 + roff);
        tile_end();
    }
}

// Skinny variant for the canvas-size projections (Q/K/V, O, W_sc): a
// 256 x 64 output tile per workgroup, four waves of 64 x 64, the same
// four-stage direct-to-LDS ring over row-major operands, split-K partials
// out (the split-K pass applies the projection's epilogue).  Two workgroups
// fit per CU (80 KiB of LDS each).
constexpr int SBN = 64;
constexpr int SA_BYTES = BM * BK * 2;    // 16 KiB
constexpr int SB_BYTES = SBN * BK * 2;   // 4 KiB

__global__ __launch_bounds__(256) void gemm_dma_skinny_kernel(GemmArgs g) {
    __shared__ __align__(1024) unsigned char a0[SA_BYTES], b0[SB_BYTES];
    __shared__ __align__(1024) unsigned char a1[SA_BYTES], b1[SB_BYTES];
    __shared__ __align__(1024) unsigned char a2[SA_BYTES], b2[SB_BYTES];
    __shared__ __align__(1024) unsigned char a3[SA_BYTES], b3[SB_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;                 // 64-row band of the tile
    const int r16 = lane & 15, g4 = lane >> 4;
    const int n0 = blockIdx.x * SBN;
    const int m0 = blockIdx.y * BM;
    const int kz = blockIdx.z;
    const int kbeg = kz * g.k_split;
    const int kend = min(g.K, kbeg + g.k_split);
    const int n = __builtin_amdgcn_readfirstlane(kend > kbeg ? (kend - kbeg) / BK : 0);

    const bf16_t* A = reinterpret_cast<const bf16_t*>(g.A);
    const int pr = lane >> 2;
    const int pc = ((lane & 3) ^ swz(pr)) * 8;
    // this wave fills A blocks 4*wave .. 4*wave+3 and B block `wave`
    const bf16_t* pa[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const long r = min(m0 + (4 * wave + q) * 16 + pr, g.M - 1);
        pa[q] = A + r * g.lda + kbeg + pc;
    }
    const long brow = min(n0 + wave * 16 + pr, g.N - 1);
    const bf16_t* pb = b_row<bf16_t>(g, (int)brow) + kbeg + pc;

#define SK_ISSUE(s, SA, SB)                                                                      \
    {                                                                                            \
        const int k_ = (s) * BK;                                                                 \
        _Pragma("unroll") for (int q = 0; q < 4; ++q)                                            \
            __builtin_amdgcn_global_load_lds((glb_void*)(pa[q] + k_),                            \
                                             (lds_void*)((SA) + (4 * wave + q) * 1024), 16, 0, 0); \
        __builtin_amdgcn_global_load_lds((glb_void*)(pb + k_), (lds_void*)((SB) + wave * 1024),  \
                                         16, 0, 0);                                              \
    }

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int roff = r16 * 64 + ((g4 ^ swz(r16)) << 4);
#define SK_COMPUTE(SA, SB)                                                                       \
    {                                                                                            \
        u32x4 f0, f1, f2, f3, e0, e1, e2, e3;                                                    \
        const uint32_t qa_ = lds_addr(SA) + wave * 4096 + roff, qb_ = lds_addr(SB) + roff;       \
        asm volatile(                                                                            \
            "ds_read_b128 %0, %8 offset:0\n ds_read_b128 %1, %8 offset:1024\n"                    \
            "ds_read_b128 %2, %8 offset:2048\n ds_read_b128 %3, %8 offset:3072\n"                 \
            "ds_read_b128 %4, %9 offset:0\n ds_read_b128 %5, %9 offset:1024\n"                    \
            "ds_read_b128 %6, %9 offset:2048\n ds_read_b128 %7, %9 offset:3072\n"                 \
            "s_waitcnt lgkmcnt(0)"                                                                \
            : "=&v"(f0), "=&v"(f1), "=&v"(f2), "=&v"(f3), "=&v"(e0), "=&v"(e1), "=&v"(e2),        \
              "=&v"(e3)                                                                          \
            : "v"(qa_), "v"(qb_)                                                                 \
            : "memory");                                                                         \
        const u32x4 fa_[4] = {f0, f1, f2, f3};                                                   \
        const u32x4 fb_[4] = {e0, e1, e2, e3};                                                   \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                            \
            _Pragma("unroll") for (int j = 0; j < 4; ++j)                                        \
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                             \
                    __builtin_bit_cast(bf16x8_t, fb_[j]), __builtin_bit_cast(bf16x8_t, fa_[i]),  \
                    acc[i][j], 0, 0, 0);                                                         \
    }
#define SK_STAGE(t, CA, CB, NA, NB)          \
    {                                        \
        if ((t) + 2 < n)                     \
            DG_WAIT_VM(10);                  \
        else if ((t) + 1 < n)                \
            DG_WAIT_VM(5);                   \
        else                                 \
            DG_WAIT_VM(0);                   \
        barrier_lds();                       \
        if ((t) + 3 < n) SK_ISSUE((t) + 3, NA, NB); \
        SK_COMPUTE(CA, CB);                  \
    }

    if (n > 0) SK_ISSUE(0, a0, b0);
    if (n > 1) SK_ISSUE(1, a1, b1);
    if (n > 2) SK_ISSUE(2, a2, b2);
    for (int t = 0; t < n; t += 4) {
        SK_STAGE(t, a0, b0, a3, b3);
        SK_STAGE(t + 1, a1, b1, a0, b0);
        SK_STAGE(t + 2, a2, b2, a1, b1);
        SK_STAGE(t + 3, a3, b3, a2, b2);
    }
#undef SK_STAGE
#undef SK_COMPUTE
#undef SK_ISSUE

    // split-K partial: lane holds row 16i + r16, columns 16j + 4*g4 .. +3
    float* C = reinterpret_cast<float*>(g.C) + (long)kz * g.M * g.ldc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + wave * 64 + 16 * i + r16;
        if (row >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + 16 * j + 4 * g4;
            if (col < g.N) *reinterpret_cast<f32x4_t*>(C + (long)row * g.ldc + col) = acc[i][j];
        }
    }
}

}  // namespace

bool gemm_dma_ok(const GemmArgs& g, int epi) {
    if (epi != EPI_STORE_F32 && epi != EPI_SPLITK) return false;
    if (g.a_rows || g.M <= 0 || g.N <= 0) return false;
    if (g.rowmax && (epi != EPI_STORE_F32 || g.N % 64)) return false;
    // whole rings of four stages in every k-range
    if (g.K % (4 * BK) || g.k_split % (4 * BK)) return false;
    if ((!g.a_tiled && g.lda % 8) || (!g.b_tiled && g.ldb % 8)) return false;
    if ((g.a_tiled || g.b_tiled) && g.K % 32) return false;
    if (g.a_tiled == 2 && (g.K % 64 || g.k_split % 64)) return false;
    // four-column stores of the output
    if (g.N % 4 || g.ldc % 4 || ((uintptr_t)g.C & 15)) return false;
    if (((uintptr_t)g.A | (uintptr_t)g.B) & 15) return false;
    return true;
}

// compute units of the current device (cached per device)
int cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cache[dev] = v;
    }
    return cache[dev];
}

hipError_t gemm_dma_bf16(const GemmArgs& g, int epi, int splits, hipStream_t st) {
    if (!gemm_dma_ok(g, epi)) return hipErrorInvalidValue;
    if (epi == EPI_STORE_F32 && g.a_tiled == 1 && g.b_tiled == 1 && splits == 1 &&
        g.N % BN == 0 && g.k_split >= g.K) {
        // one workgroup per CU (the ring fills 128 KiB of LDS), a whole
        // number per XCD, the row tiles of a column tile on one XCD
        const int rt = cdiv(g.M, BM);
        const int slots = std::max(1, cu_count() / 8);
        if (rt <= slots) {
            hipLaunchKernelGGL(gemm_head_kernel<4>, dim3(8 * slots), dim3(WAVES * 64), 0, st, g, rt);
            return hipGetLastError();
        }
    }
    dim3 grid(cdiv(g.N, BN), cdiv(g.M, BM), splits);
    // The head's weight (E, 1 GB) is streamed once: its loads are
    // non-temporal (measured 299 -> 284 us for the full-vocabulary head;
    // the same hint on the self-conditioning product's E^T was slower).
    // (a ring of five stages, all of LDS, measured slower than four: 289
    // against 282 us on the head)
#define DG_LAUNCH(E, TA_, TB_)                                                                 \
    hipLaunchKernelGGL((gemm_dma_kernel<E, TA_, TB_, (E == EPI_STORE_F32 && TB_) ? 2 : 0, 4>), \
                       grid, dim3(WAVES * 64), 0, st, g)
    if (g.a_tiled == 2) {   // 64-wide blocked A (the self-conditioning operand)
        if (epi != EPI_SPLITK || !g.b_tiled) return hipErrorInvalidValue;
        DG_LAUNCH(EPI_SPLITK, 2, 1);
        return hipGetLastError();
    }
    const int t = (g.a_tiled ? 1 : 0) | (g.b_tiled ? 2 : 0);
    if (epi == EPI_STORE_F32) {
        if (t == 3) DG_LAUNCH(EPI_STORE_F32, 1, 1);
        else if (t == 0) DG_LAUNCH(EPI_STORE_F32, 0, 0);
        else return hipErrorInvalidValue;
    } else {
        if (t == 3) DG_LAUNCH(EPI_SPLITK, 1, 1);
        else if (t == 0) DG_LAUNCH(EPI_SPLITK, 0, 0);
        else return hipErrorInvalidValue;
    }
#undef DG_LAUNCH
    return hipGetLastError();
}

bool gemm_skinny_ok(const GemmArgs& g) {
    if (g.a_rows || g.M <= 0 || g.N <= 0 || g.a_tiled || g.b_tiled) return false;
    if (g.K % (4 * BK) || g.k_split % (4 * BK)) return false;
    if (g.lda % 8 || g.ldb % 8 || g.N % 4 || g.ldc % 4) return false;
    if (((uintptr_t)g.A | (uintptr_t)g.B | (uintptr_t)g.C) & 15) return false;
    if ((g.B2 && ((uintptr_t)g.B2 & 15)) || (g.B3 && ((uintptr_t)g.B3 & 15))) return false;
    return true;
}

hipError_t gemm_skinny_splitk(const GemmArgs& g, int splits, hipStream_t st) {
    if (!gemm_skinny_ok(g)) return hipErrorInvalidValue;
    dim3 grid(cdiv(g.N, SBN), cdiv(g.M, BM), splits);
    hipLaunchKernelGGL(gemm_dma_skinny_kernel, grid, dim3(256), 0, st, g);
    return hipGetLastError();
}

}  // namespace dg
