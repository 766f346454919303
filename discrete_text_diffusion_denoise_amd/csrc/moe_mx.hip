// Quantised expert GEMMs on gfx950's block-scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4): the weight codes -- MXFP4 (E2M1 with
// an E8M0 scale per 32 k) or E4M3 with one fp32 scale per row -- and the
// MXFP8 token activations (E4M3 with an E8M0 scale per 32 features) enter
// the matrix cores as they are stored; nothing is widened in registers.
//
// youleyou.com article, "Deployment": the model ships tuned for a 4-bit
// floating-point weight format so that the memory-bound mixture of experts
// moves fewer bytes; report-summary page (animattoys.com), section 5: the
// canvas step is bound by loading expert weights.  So every weight byte of a
// hit expert is streamed once per chunk of up to 32 of its tokens, in whole
// 128-byte lines.
//
// Operand layout of one 16x16x128 step (measured on gfx950 with random codes
// and scales, every product checked): A (16 weight rows) -- lane l holds row
// l % 16; E2M1: 16 bytes, k = 32 (l / 16) .. +31, the even k in the low
// nibble; E4M3: 32 bytes, k = 16 (l / 16) .. +15 then 64 + 16 (l / 16) ..
// +15.  B (16 tokens) -- lane l holds token l % 16 in the E4M3 layout.  The
// scale operand of lane l is the E8M0 code of (row or token l % 16, 32-k
// block l / 16).  Output: lane l holds rows 4 (l / 16) + i of the tile for
// token l % 16.  The quantisers store the weights tiled in exactly this lane
// order (dg_quantize_mxfp4 / dg_quantize_fp8), so one 16-row tile's step is
// 1 KiB (E4M3: two) that a wave copies with one 1-KiB load and reads back
// as its operand with one conflict-free 16-byte LDS read per lane.
//
// Work split: a wave owns 16 output features (MODE 0: a gate tile and the up
// tile of the same features) or 32 rows of W_down (MODE 1); a workgroup of
// four waves shares the token chunk.  Weight tiles, their scale codes, token
// rows and token scale codes of each 128-k step go by direct-to-LDS loads
// into a ring of D + 1 slots, D steps ahead; one wait per step (for the step
// issued D steps earlier) leaves the later D - 1 steps in flight.  The
// gate/up epilogue forms silu(gate) * up in fp32 and writes it as MXFP8 for
// the down product: the two waves holding a 32-feature block trade their
// partial maxima through LDS.
#include "common.h"
#include "kernels.h"
#include "lds_ring.h"
#include "mx.h"

#include <algorithm>

namespace dg {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int MX_TOK_BYTES = 32 * 128;    // token codes of a slot (32 rows of 128 k)
constexpr int MX_TSC_BYTES = 4 * 256;     // token scale codes of a slot: a copy per wave

// Keeps the memory operations on either side in program order, for the
// compiler and for the instruction scheduler: the vmcnt arithmetic below
// counts issues in the order written.
__device__ __forceinline__ void issue_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// bytes of one ring slot: weight tiles (8 per workgroup), their scale codes
// (MXFP4: 256 bytes a tile), token codes and token scale codes
template <int WF>
constexpr int mx_slot_bytes() {
    return 8 * (WF == 0 ? 1024 : 2048) + (WF == 0 ? 8 * 256 : 0) + MX_TOK_BYTES + MX_TSC_BYTES;
}

struct MxCtx {
    int e, off, cnt, K, NOUT, S;       // S = K / 128 steps
    int lane, wave, t16, g;
    int f0;                            // MODE 0: first feature of the wave; MODE 1: first row
    int c0;                            // the chunk's first token (of the expert's cnt)
    const uint8_t* wt[2];              // this wave's weight tiles 0 and 1 at step 0
    const uint8_t* xt[2];              // MXFP4: their scale codes at step 0
    const uint8_t* X8;                 // token codes [rows][K]
    const uint8_t* X8s;                // token scale codes [rows][K / 32]
};

template <int MODE, int WF, int TT, int D>
__device__ __forceinline__ void mx_body(const MoeArgs& a, const MxCtx& c, unsigned char* lds,
                                        float* xch) {
    static_assert(TT == 1 || TT == 2, "chunks of at most 32 tokens");
    static_assert(D >= 1, "pipeline depth");
    constexpr int WT = WF == 0 ? 1024 : 2048;       // bytes of one tile-step
    constexpr int NWD = WT / 1024;                  // its 1-KiB loads
    constexpr int NSD = WF == 0 ? 2 : 0;            // weight scale-code loads per wave and step
    constexpr int ND = 2 * NWD + NSD + 2;           // loads per wave and step (+ token codes, scales)
    constexpr int NS = D + 1;                       // ring slots
    constexpr int SLOT = mx_slot_bytes<WF>();
    // slot layout: weight tiles [wave][tile], their scale codes, token rows, token scales
    constexpr int O_WS = 8 * WT, O_TOK = O_WS + (WF == 0 ? 8 * 256 : 0), O_TSC = O_TOK + MX_TOK_BYTES;
    const int S = c.S;
    const int lane = c.lane, wave = c.wave, t16 = c.t16, g = c.g;

    // per-row fp32 scales of E4M3 weights (rows 4g .. 4g+3 of each tile)
    f32x4_t rs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        rs[j] = f32x4_t{1.f, 1.f, 1.f, 1.f};
        if (WF == 1) {
            const float* sv = MODE == 0 ? (j == 0 ? a.s_gate : a.s_up) : a.s_down;
            const int r0 = MODE == 0 ? c.f0 : c.f0 + 16 * j;
            rs[j] = *reinterpret_cast<const f32x4_t*>(sv + (long)c.e * c.NOUT + r0 + 4 * g);
        }
    }
    const uint32_t lds_l = lds_addr(lds);
    // fragment addresses in slot 0: this wave's weight tiles (16 bytes a
    // lane, in lane order), their scale codes (a byte a lane), token row t16
    // of tile 0 (tile tt is 2 KiB further), its chunks g and 4 + g (16-byte
    // chunk q of token row r sits in place q ^ (r & 7)), and its scale code
    // of block g
    const uint32_t fw = lds_l + (2 * wave) * WT + 16 * lane;
    const uint32_t fws = lds_l + O_WS + (2 * wave) * 256 + lane;
    const uint32_t fa0 = lds_l + O_TOK + t16 * 128 + ((g ^ (t16 & 7)) << 4);
    const uint32_t fa1 = lds_l + O_TOK + t16 * 128 + (((4 + g) ^ (t16 & 7)) << 4);
    const uint32_t fsc = lds_l + O_TSC + wave * 256 + t16 * 4 + g;

    const int c0 = c.c0;
    // token loads: this wave fills token rows 8 wave .. +7 of the slot (lane
    // l: row + l / 8, place l % 8 holding chunk (l % 8) ^ (row & 7)), and
    // copies the scale codes of all 32 rows (lane l: row min(l, 31)) into its
    // own 256 bytes.  Rows past the chunk's tokens repeat its last token.
    const uint8_t* tsrc;
    {
        const int r = 8 * wave + (lane >> 3);
        const int tr = min(c0 + r, c.cnt - 1);
        const long row = MODE == 0 ? (long)a.perm_tok[c.off + tr] : (long)(c.off + tr);
        tsrc = c.X8 + row * c.K + 16 * ((lane & 7) ^ (r & 7));
    }
    const uint8_t* ssrc;
    {
        const int tr = min(c0 + min(lane, 31), c.cnt - 1);
        const long row = MODE == 0 ? (long)a.perm_tok[c.off + tr] : (long)(c.off + tr);
        ssrc = c.X8s + row * (c.K / 32);
    }
    // All loads of a step, unconditionally; a step past the end loads step
    // S - 1 again (into a slot no later step reads), so every step issues the
    // same operations and the wait count is a constant.  The weight scale
    // codes (64 bytes a tile-step) are copied four times over 256 bytes, so
    // every lane of the load has a place.
    auto issue = [&](int s, int slot) {
        s = min(s, S - 1);
        unsigned char* sl = lds + slot * SLOT;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < NWD; ++h)
                __builtin_amdgcn_global_load_lds(
                    (glb_void*)(c.wt[j] + (long)s * WT + h * 1024 + 16 * lane),
                    (lds_void*)(sl + (2 * wave + j) * WT + h * 1024), 16, 0, 0);
        if (WF == 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                __builtin_amdgcn_global_load_lds((glb_void*)(c.xt[j] + (long)s * 64 + 4 * (lane & 15)),
                                                 (lds_void*)(sl + O_WS + (2 * wave + j) * 256), 4, 0, 0);
        }
        __builtin_amdgcn_global_load_lds((glb_void*)(tsrc + 128L * s),
                                         (lds_void*)(sl + O_TOK + (8 * wave) * 128), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void*)(ssrc + 4 * s),
                                         (lds_void*)(sl + O_TSC + wave * 256), 4, 0, 0);
    };
    f32x4_t acc[2][TT];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[j][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // prologue: steps 0 .. D-1
#pragma unroll
    for (int x = 0; x < D; ++x) {
        issue(x, x);
        issue_fence();
    }
    // step s: wait for its loads (issued D steps earlier; after them, D - 1
    // steps' worth), every wave past the barrier, refill the slot read one
    // step ago with step s + D, multiply.  slot = s mod (D + 1).
    int slot = 0;
    for (int s = 0; s < S; ++s) {
        issue_fence();
        DG_WAIT_VM((D - 1) * ND);
        barrier_lds();
        issue(s + D, slot == 0 ? NS - 1 : slot - 1);
        issue_fence();
        const uint32_t o = slot * SLOT;
        slot = slot + 1 == NS ? 0 : slot + 1;
        u32x4 wa[2], wb[2], fa[TT], fb[TT];
        uint32_t ws[2], fs[TT];
        // weight operands (E4M3: both 1-KiB halves) and scale codes
        if (WF == 0) {
            asm volatile(
                "ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:1024\n"
                "ds_read_u8 %2, %5\n ds_read_u8 %3, %5 offset:256\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(wa[0]), "=&v"(wa[1]), "=&v"(ws[0]), "=&v"(ws[1])
                : "v"(fw + o), "v"(fws + o)
                : "memory");
            wb[0] = wb[1] = u32x4{0u, 0u, 0u, 0u};
        } else {
            asm volatile(
                "ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:1024\n"
                "ds_read_b128 %2, %4 offset:2048\n ds_read_b128 %3, %4 offset:3072\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(wa[0]), "=&v"(wb[0]), "=&v"(wa[1]), "=&v"(wb[1])
                : "v"(fw + o)
                : "memory");
            ws[0] = ws[1] = 127u;
        }
        if (TT == 1) {
            asm volatile(
                "ds_read_b128 %0, %3\n ds_read_b128 %1, %4\n ds_read_u8 %2, %5\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(fa[0]), "=&v"(fb[0]), "=&v"(fs[0])
                : "v"(fa0 + o), "v"(fa1 + o), "v"(fsc + o)
                : "memory");
        } else {
            asm volatile(
                "ds_read_b128 %0, %6\n ds_read_b128 %1, %7\n"
                "ds_read_b128 %2, %6 offset:2048\n ds_read_b128 %3, %7 offset:2048\n"
                "ds_read_u8 %4, %8\n ds_read_u8 %5, %8 offset:64\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(fa[0]), "=&v"(fb[0]), "=&v"(fa[TT - 1]), "=&v"(fb[TT - 1]), "=&v"(fs[0]),
                  "=&v"(fs[TT - 1])
                : "v"(fa0 + o), "v"(fa1 + o), "v"(fsc + o)
                : "memory");
        }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const i32x8_t A = {(int)wa[jt][0], (int)wa[jt][1], (int)wa[jt][2], (int)wa[jt][3],
                               (int)wb[jt][0], (int)wb[jt][1], (int)wb[jt][2], (int)wb[jt][3]};
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const i32x8_t B = {(int)fa[tt][0], (int)fa[tt][1], (int)fa[tt][2], (int)fa[tt][3],
                                   (int)fb[tt][0], (int)fb[tt][1], (int)fb[tt][2], (int)fb[tt][3]};
                acc[jt][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    A, B, acc[jt][tt], WF == 0 ? 4 : 0, 0, 0, (int)ws[jt], 0, (int)fs[tt]);
            }
        }
    }
    // the loads of steps past the end are still in flight: none may land in
    // the ring after the workgroup has left it
    DG_WAIT_VM(0);

    if constexpr (MODE == 0) {
        // silu(gate) * up of features f0 + 4g + i, token 16 tt + t16; the
        // block of 32 features is this wave's 16 and its partner's (wave ^ 1)
        float v[TT][4];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gv = acc[0][tt][i] * rs[0][i];
                const float uv = acc[1][tt][i] * rs[1][i];
                v[tt][i] = gv / (1.0f + __expf(-gv)) * uv;
                m = fmaxf(m, fabsf(v[tt][i]));
            }
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            if (g == 0) xch[wave * 64 + 16 * tt + t16] = m;
        }
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int r = c0 + 16 * tt + t16;
            const float m = fmaxf(xch[wave * 64 + 16 * tt + t16], xch[(wave ^ 1) * 64 + 16 * tt + t16]);
            const int ex = mx8_exponent(m);
            const float inv = __builtin_amdgcn_ldexpf(1.0f, -ex);
            if (r < c.cnt) {
                const long arow = c.off + r;
                const uint32_t code = e4m3_act(v[tt][0] * inv) | (e4m3_act(v[tt][1] * inv) << 8) |
                                      (e4m3_act(v[tt][2] * inv) << 16) |
                                      (e4m3_act(v[tt][3] * inv) << 24);
                *reinterpret_cast<uint32_t*>(a.act8 + arow * a.F + c.f0 + 4 * g) = code;
                if (g == 0 && (wave & 1) == 0)
                    a.act8s[arow * (a.F / 32) + c.f0 / 32] = (uint8_t)(ex + 127);
            }
        }
    } else {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int r = c0 + 16 * tt + t16;
            if (r >= c.cnt) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const f32x4_t y = acc[j][tt] * rs[j];
                *reinterpret_cast<f32x4_t*>(a.y + (long)(c.off + r) * a.d + c.f0 + 16 * j + 4 * g) = y;
            }
        }
    }
}

// blockIdx.x: 64 features (MODE 0) or 128 rows of W_down (MODE 1);
// blockIdx.y: a work item, one chunk of up to 32 tokens of one expert, the
// busiest experts' chunks first (work[] over order[], from the routing), so a
// busy expert's chunks run side by side and share its weight stream through
// the caches.  WF: 0 MXFP4 weights, 1 E4M3 weights with per-row scales.
template <int MODE, int WF, int D>
__global__ __launch_bounds__(256) void expert_mx_kernel(MoeArgs a) {
    if (a.halt && *a.halt) return;
    const int w = blockIdx.y;
    if (w >= a.work[a.E]) return;
    __shared__ __align__(1024) unsigned char lds[(D + 1) * mx_slot_bytes<WF>()];
    __shared__ float xch[4 * 64];
    // the rank r of the item's expert: work[r] <= w < work[r + 1]
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.work[mid] <= w)
            lo = mid;
        else
            hi = mid - 1;
    }
    MxCtx c;
    c.e = a.order[lo];
    c.off = a.offsets[c.e];
    c.c0 = (w - a.work[lo]) * kMoeChunk;
    c.cnt = a.offsets[c.e + 1] - c.off;
    const int tid = threadIdx.x;
    c.lane = tid & 63;
    c.wave = tid >> 6;
    c.t16 = c.lane & 15;
    c.g = c.lane >> 4;
    c.K = MODE == 0 ? a.d : a.F;
    c.NOUT = MODE == 0 ? a.F : a.d;
    c.S = __builtin_amdgcn_readfirstlane(c.K / 128);
    c.f0 = MODE == 0 ? blockIdx.x * 64 + 16 * c.wave : blockIdx.x * 128 + 32 * c.wave;
    constexpr int WT = WF == 0 ? 1024 : 2048;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint8_t* W = reinterpret_cast<const uint8_t*>(
            MODE == 0 ? (j == 0 ? a.w_gate : a.w_up) : a.w_down);
        // tiles of 16 rows, each a run of S tile-steps
        const long tile = ((long)c.e * c.NOUT + (MODE == 0 ? c.f0 : c.f0 + 16 * j)) / 16;
        c.wt[j] = W + tile * c.S * WT;
        c.xt[j] = nullptr;
        if (WF == 0) {
            const uint8_t* X = MODE == 0 ? (j == 0 ? a.x_gate : a.x_up) : a.x_down;
            c.xt[j] = X + tile * c.S * 64;
        }
    }
    c.X8 = MODE == 0 ? a.u8 : a.act8;
    c.X8s = MODE == 0 ? a.u8s : a.act8s;
    const int rows = __builtin_amdgcn_readfirstlane(min(c.cnt - c.c0, kMoeChunk));
    if (rows <= 16)
        mx_body<MODE, WF, 1, D>(a, c, lds, xch);
    else
        mx_body<MODE, WF, 2, D>(a, c, lds, xch);
}

// One launch per product; grid.y covers the most work items there can be
// (every expert's last chunk partial).  Steps in flight: MXFP4 4 (five slots
// of 15 KiB: two workgroups a CU, 32 KiB of weights in flight each), E4M3 2
// (three slots of 21 KiB: the same).
template <int MODE, int WF>
void launch_mx(const MoeArgs& a, int blocks, hipStream_t st) {
    const dim3 grid(blocks, cdiv(a.T * a.k, kMoeChunk) + std::min(a.E, a.T * a.k));
    hipLaunchKernelGGL((expert_mx_kernel<MODE, WF, WF == 0 ? 4 : 2>), grid, dim3(256), 0, st, a);
}

}  // namespace

// the block-scaled kernels' shape limits: 64 features per workgroup of the
// gate/up product, 128 rows of the down product, 128 k per step
bool expert_mx_ok(const MoeArgs& a) {
    return a.F % 128 == 0 && a.d % 128 == 0 && a.u8 && a.u8s && a.act8 && a.act8s && a.order &&
           a.work &&
           (a.f4 ? (a.x_gate && a.x_up && a.x_down)
                 : (a.f8 && a.s_gate && a.s_up && a.s_down));
}

hipError_t moe_gateup_mx(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (!expert_mx_ok(a)) return hipErrorInvalidValue;
    if (a.f4)
        launch_mx<0, 0>(a, a.F / 64, st);
    else
        launch_mx<0, 1>(a, a.F / 64, st);
    return hipGetLastError();
}

hipError_t moe_down_mx(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (!expert_mx_ok(a)) return hipErrorInvalidValue;
    if (a.f4)
        launch_mx<1, 0>(a, a.d / 128, st);
    else
        launch_mx<1, 1>(a, a.d / 128, st);
    return hipGetLastError();
}

}  // namespace dg
