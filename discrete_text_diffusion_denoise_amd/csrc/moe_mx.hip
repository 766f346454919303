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
// hit expert is streamed once per chunk of up to 64 of its tokens, in whole
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
// Work split: a task is one row block of one work item (a chunk of up to 64
// tokens of one expert); a wave owns 16 output features (MODE 0: a gate tile
// and the up tile of the same features) or 32 rows of W_down (MODE 1), and a
// workgroup of four waves shares the token chunk.  The grid is persistent:
// each workgroup runs its tasks back to back through one ring of D + 1 LDS
// slots, into which every 128-k step's weight tiles, scale codes, token rows
// and token scale codes go by direct-to-LDS loads, D steps ahead and across
// task boundaries, so the ring fills once per workgroup, not once per task.
// One wait per step (for the step issued D steps earlier) leaves the later
// D - 1 steps in flight; nothing inside the stream waits for all loads.  The
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
typedef __attribute__((address_space(4))) const int32_t c_i32;

// A load through the scalar data cache (the address must be uniform): its
// wait is lgkmcnt, so it never holds up the ring's vector-memory count.
// The arrays read this way (routing tables) are not written by the kernels
// that read them.
__device__ __forceinline__ int sload(const int32_t* p) { return *(const c_i32*)p; }

// Keeps the memory operations on either side in program order, for the
// compiler and for the instruction scheduler: the vmcnt arithmetic below
// counts issues in the order written.
__device__ __forceinline__ void issue_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

constexpr int MX_TPW = 2;                 // weight tiles (16 rows each) a wave streams
constexpr int MX_TOK_BYTES = kMoeChunk * 128;   // token codes of a 128-k step (64 rows)
template <int WF>
constexpr int mx_tile_bytes() { return WF == 0 ? 1024 : 2048; }   // one tile's 128-k step
// steps in flight: two, in rings of three slots (MXFP4 17 KiB a slot: three
// workgroups a CU, 51 KiB each; E4M3 25 KiB: two)
template <int WF>
constexpr int mx_depth() { return 2; }

// one ring slot: the workgroup's weight tiles [wave][tile]; a 256-byte
// auxiliary region per wave: bytes 0..127 its tiles' bytes (MXFP4: their
// scale codes; E4M3: their rows' fp32 scales), 128..159 the scale codes of
// token rows 8 wave .. +7, 160..191 of rows 32 + 8 wave .. +7 (192..255 a
// repeat); the 64 token rows
template <int WF>
struct MxSlot {
    static constexpr int W = 4 * MX_TPW * mx_tile_bytes<WF>();
    static constexpr int AUX = W;
    static constexpr int TOK = AUX + 4 * 256;
    static constexpr int BYTES = TOK + MX_TOK_BYTES;
};
template <int WF>
constexpr int mx_lds_bytes() {
    return (mx_depth<WF>() + 1) * MxSlot<WF>::BYTES;
}

// the uniform part of a task: its expert, the expert's rows in the sorted
// order, the chunk's first token, this wave's first feature (MODE 0) or row
// (MODE 1)
struct MxTask {
    int e, off, cnt, c0, f0;
};

template <int MODE>
__device__ __forceinline__ MxTask mx_task(const MoeArgs& a, int t, int NX, int wave) {
    const int w = t / NX, bx = t - w * NX;
    MxTask k;
    if (a.items) {
        // the item's record: one scalar load of four words
        const int32_t* rec = a.items + 4 * w;
        k.e = sload(rec);
        k.off = sload(rec + 1);
        k.c0 = sload(rec + 2);
        k.cnt = sload(rec + 3);
    } else {
        // the rank r of the item's expert (work[r] <= w < work[r + 1])
        int lo = 0, hi = a.E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sload(a.work + mid) <= w)
                lo = mid;
            else
                hi = mid - 1;
        }
        k.e = sload(a.order + lo);
        k.off = sload(a.offsets + k.e);
        k.cnt = sload(a.offsets + k.e + 1) - k.off;
        k.c0 = (w - sload(a.work + lo)) * kMoeChunk;
    }
    k.f0 = MODE == 0 ? bx * (32 * MX_TPW) + 16 * (MX_TPW / 2) * wave
                     : bx * (64 * MX_TPW) + 16 * MX_TPW * wave;
    return k;
}


// where a task's loads come from (step 0): the wave's weight tile runs, and
// per lane its auxiliary bytes, token codes and token scale codes
struct MxSrc {
    const uint8_t* wt[MX_TPW];
    const uint8_t* aux;     // per lane: lanes 0..31 the tiles' bytes, 32..63 token scale codes
    int astep;              // its advance per step
    const uint8_t* tok[2];  // per lane: its token row of each of the wave's two loads
    bool big;               // more than 32 tokens: the second token load too
};

template <int MODE, int WF>
__device__ __forceinline__ MxSrc mx_src(const MoeArgs& a, const MxTask& k, int lane, int wave,
                                        int K, int NOUT, int S) {
    constexpr int HALF = MX_TPW / 2;
    constexpr int WT = mx_tile_bytes<WF>();
    MxSrc r;
#pragma unroll
    for (int j = 0; j < MX_TPW; ++j) {
        const uint8_t* W =
            reinterpret_cast<const uint8_t*>(MODE == 0 ? (j < HALF ? a.w_gate : a.w_up) : a.w_down);
        const int r0 = MODE == 0 ? k.f0 + 16 * (j % HALF) : k.f0 + 16 * j;
        r.wt[j] = W + ((long)k.e * NOUT + r0) / 16 * S * WT;   // tiles of 16 rows, S steps each
    }
    // auxiliary region: lane l copies 4 bytes of tile jl = (l / 16) mod TPW
    // (a repeat past the wave's tiles); MXFP4: that tile's 64 scale bytes of
    // the step; E4M3: its 16 rows' scales (the same every step)
    {
        const int jl = (lane >> 4) % MX_TPW;
        const int r0 = MODE == 0 ? k.f0 + 16 * (jl % HALF) : k.f0 + 16 * jl;
        const long tile = ((long)k.e * NOUT + r0) / 16;
        if (WF == 0) {
            const uint8_t* X = MODE == 0 ? (jl < HALF ? a.x_gate : a.x_up) : a.x_down;
            r.aux = X + tile * S * 64 + 4 * (lane & 15);
            r.astep = 64;
        } else {
            const float* sv = MODE == 0 ? (jl < HALF ? a.s_gate : a.s_up) : a.s_down;
            r.aux = reinterpret_cast<const uint8_t*>(sv + tile * 16 + (lane & 15));
            r.astep = 0;
        }
    }
    // the wave's token rows 8 wave .. +7 and 32 + 8 wave .. +7 of the chunk
    // (rows past the expert's tokens repeat its last one); load q of lane l
    // takes row 32 q + 8 wave + l / 8, 16-byte chunk (l % 8) ^ (l / 8 % 8) of
    // the step (load 1 only for chunks of more than 32 tokens); lanes
    // 32 + 8 q + i (and 48 + 8 q + i) the scale codes of row 32 q + 8 wave + i
    r.big = k.cnt - k.c0 > 32;
    int base[2], it[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        base[q] = min(k.c0 + 32 * q + 8 * wave, k.cnt - 1);
        it[q] = 8 * q + min(k.c0 + 32 * q + 8 * wave + (lane >> 3), k.cnt - 1) - base[q];
    }
    const int qs = (lane >> 3) & 1;
    const int is = 8 * qs + min(k.c0 + 32 * qs + 8 * wave + (lane & 7), k.cnt - 1) - (qs ? base[1] : base[0]);
    long row_t[2], row_s;
    if (MODE == 0) {
        // the 16 sorted slots' tokens (8 from each base) by scalar loads
        // (perm_tok has 16 entries of padding past its end), written into
        // lanes 0..15 and picked per lane by a cross-lane read (an array
        // indexed per lane would go to scratch memory)
        int pv = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int v = sload(a.perm_tok + k.off + base[i >> 3] + (i & 7));
            if (lane == i) pv = v;
        }
        row_t[0] = __shfl(pv, it[0], 64);
        row_t[1] = __shfl(pv, it[1], 64);
        row_s = __shfl(pv, is, 64);
    } else {
        row_t[0] = k.off + base[0] + it[0];
        row_t[1] = k.off + base[1] + it[1] - 8;
        row_s = k.off + (qs ? base[1] : base[0]) + is - 8 * qs;
    }
    const uint8_t* X8 = MODE == 0 ? a.u8 : a.act8;
    const uint8_t* X8s = MODE == 0 ? a.u8s : a.act8s;
#pragma unroll
    for (int q = 0; q < 2; ++q) r.tok[q] = X8 + row_t[q] * K + 16 * ((lane & 7) ^ ((lane >> 3) & 7));
    if (lane >= 32) {
        r.aux = X8s + row_s * (K / 32);
        r.astep = 4;
    }
    return r;
}

// Persistent: workgroup b runs tasks b, b + G, b + 2G, ... of the NX x
// work[E] tasks (G: the workgroups the rounds need, at most gridDim.x), task
// t = (work item t / NX, row block t % NX); the work items are the busiest
// experts' chunks first (work[] over order[], from the routing).  Row blocks
// of 32 TPW features (MODE 0) or 64 TPW rows of W_down (MODE 1).  WF: 0
// MXFP4 weights, 1 E4M3 weights with per-row scales.
template <int MODE, int WF>
__global__ __launch_bounds__(256) void expert_mx_kernel(MoeArgs a, int cus) {
    if (a.halt && *a.halt) return;
    constexpr int D = mx_depth<WF>();
    constexpr int TPW = MX_TPW;
    constexpr int WT = mx_tile_bytes<WF>();
    constexpr int NWD = WT / 1024;                  // 1-KiB loads of a tile-step
    // loads per wave and step (a step of a chunk of more than 32 tokens: one
    // more; the wait below counts the fewer, so such a step only waits a
    // little longer than it must)
    constexpr int ND = TPW * NWD + 2;
    constexpr int NS = D + 1;                       // ring slots
    using L = MxSlot<WF>;
    constexpr int SLOT = L::BYTES;
    __shared__ __align__(1024) unsigned char lds[mx_lds_bytes<WF>()];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t16 = lane & 15, g = lane >> 4;
    const int K = MODE == 0 ? a.d : a.F;
    const int NOUT = MODE == 0 ? a.F : a.d;
    const int S = K / 128;
    const int NX = MODE == 0 ? a.F / (32 * TPW) : a.d / (64 * TPW);
    const int NT = sload(a.work + a.E) * NX;
    // the tasks spread evenly: as few rounds as the grid allows, and as few
    // workgroups as those rounds need, so that no workgroup runs a last task
    // alone while the others have finished
    const int rounds = cdiv(NT, (int)gridDim.x);
    const int G = rounds ? cdiv(NT, rounds) : 0, b = blockIdx.x;
    if (b >= G) return;
    const int ntask = (NT - 1 - b) / G + 1;
    // the workgroup's place among those sharing its CU (workgroups are
    // handed out to the CUs in turn): issue arbitration favours the oldest
    // wave, so a CU's first workgroup would run ahead of the later ones and
    // leave the CU with fewer loads in flight at the end; rotating the
    // priority every step evens their progress out
    constexpr int PER_CU = (160 * 1024) / mx_lds_bytes<WF>();
    const int cu_slot = b / cus;

    const uint32_t lds_l = lds_addr(lds);
    // fragment addresses in slot 0: this wave's weight tiles (16 bytes a
    // lane, in lane order; E4M3: two 1-KiB halves), their scale codes (a byte
    // a lane, 64 bytes a tile); token row t16 (row 16 tt + t16: 2 tt KiB
    // further), its chunks g and 4 + g (16-byte chunk q of token row r sits
    // in place q ^ (r & 7)); the scale code of token t16, block g (rows
    // 16 tt + t16 of tiles 1, 2, 3: 512, 32 and 544 bytes further, in the
    // regions of the waves that load them); the wave's auxiliary region
    const uint32_t fw = lds_l + (TPW * wave) * WT + 16 * lane;
    const uint32_t fws = lds_l + L::AUX + wave * 256 + lane;
    const uint32_t fa0 = lds_l + L::TOK + t16 * 128 + ((g ^ (t16 & 7)) << 4);
    const uint32_t fa1 = lds_l + L::TOK + t16 * 128 + (((4 + g) ^ (t16 & 7)) << 4);
    const uint32_t fsc = lds_l + L::AUX + (t16 >> 3) * 256 + 128 + (t16 & 7) * 4 + g;
    const uint32_t frs = lds_l + L::AUX + wave * 256 + 16 * g;

    // issue side: task ni of this workgroup, step si; every step issues the
    // same loads, so the wait count is a constant; after the last task's
    // last step it loads that step again (into slots no later step reads)
    int ni = 0, si = 0;
    MxSrc src = mx_src<MODE, WF>(a, mx_task<MODE>(a, b, NX, wave), lane, wave, K, NOUT, S);
    auto issue = [&](int slot) {
        unsigned char* sl = lds + slot * SLOT;
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int q = 0; q < NWD; ++q)
                __builtin_amdgcn_global_load_lds(
                    (glb_void*)(src.wt[j] + (long)si * WT + q * 1024 + 16 * lane),
                    (lds_void*)(sl + (TPW * wave + j) * WT + q * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void*)(src.aux + si * src.astep),
                                         (lds_void*)(sl + L::AUX + wave * 256), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void*)(src.tok[0] + 128L * si),
                                         (lds_void*)(sl + L::TOK + (8 * wave) * 128), 16, 0, 0);
        if (src.big)
            __builtin_amdgcn_global_load_lds((glb_void*)(src.tok[1] + 128L * si),
                                             (lds_void*)(sl + L::TOK + (32 + 8 * wave) * 128), 16, 0, 0);
        if (si + 1 < S) {
            ++si;
        } else if (ni + 1 < ntask) {
            ++ni;
            si = 0;
            src = mx_src<MODE, WF>(a, mx_task<MODE>(a, b + ni * G, NX, wave), lane, wave, K, NOUT, S);
        }
    };

    // compute side: task nc, step sc
    MxTask ct = mx_task<MODE>(a, b, NX, wave);
    int ntt = min(4, cdiv(ct.cnt - ct.c0, 16));     // the chunk's 16-token tiles
    f32x4_t acc[TPW][4];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[j][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int x = 0; x < D; ++x) {
        issue(x);
        issue_fence();
    }
    // step: wait for its loads (issued D steps earlier; after them, D - 1
    // steps' worth and at most a task's epilogue stores), every wave past the
    // barrier, refill the slot read one step ago, multiply; slot = step mod
    // (D + 1)
    const int steps = ntask * S;
    int slot = 0, sc = 0, nc = 0;
    for (int gs = 0; gs < steps; ++gs) {
        issue_fence();
        DG_WAIT_VM((D - 1) * ND);
        barrier_lds();
        if (PER_CU > 1) {
            const int pr = (gs + cu_slot) % PER_CU;
            if (pr == 0)
                __builtin_amdgcn_s_setprio(0);
            else if (pr == 1)
                __builtin_amdgcn_s_setprio(1);
            else if (pr == 2)
                __builtin_amdgcn_s_setprio(2);
            else
                __builtin_amdgcn_s_setprio(3);
        }
        issue(slot == 0 ? NS - 1 : slot - 1);
        issue_fence();
        const uint32_t o = slot * SLOT;
        slot = slot + 1 == NS ? 0 : slot + 1;
        u32x4 wa[TPW], wb[TPW], fa[4], fb[4];
        uint32_t ws[TPW], fs[4];
        // all fragments of the step in one LDS round trip: the weights, and
        // the token tiles 0, 1 (2, 3 too when the chunk has more than 32
        // tokens)
        if constexpr (WF == 0) {
            wb[0] = wb[1] = u32x4{0u, 0u, 0u, 0u};
            if (ntt > 2)
                asm volatile(
                    "ds_read_b128 %0, %16\n ds_read_b128 %1, %16 offset:1024\n"
                    "ds_read_u8 %2, %17\n ds_read_u8 %3, %17 offset:64\n"
                    "ds_read_b128 %4, %18\n ds_read_b128 %5, %19\n"
                    "ds_read_b128 %6, %18 offset:2048\n ds_read_b128 %7, %19 offset:2048\n"
                    "ds_read_b128 %8, %18 offset:4096\n ds_read_b128 %9, %19 offset:4096\n"
                    "ds_read_b128 %10, %18 offset:6144\n ds_read_b128 %11, %19 offset:6144\n"
                    "ds_read_u8 %12, %20\n ds_read_u8 %13, %20 offset:512\n"
                    "ds_read_u8 %14, %20 offset:32\n ds_read_u8 %15, %20 offset:544\n"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(wa[0]), "=&v"(wa[1]), "=&v"(ws[0]), "=&v"(ws[1]), "=&v"(fa[0]), "=&v"(fb[0]),
                      "=&v"(fa[1]), "=&v"(fb[1]), "=&v"(fa[2]), "=&v"(fb[2]), "=&v"(fa[3]), "=&v"(fb[3]),
                      "=&v"(fs[0]), "=&v"(fs[1]), "=&v"(fs[2]), "=&v"(fs[3])
                    : "v"(fw + o), "v"(fws + o), "v"(fa0 + o), "v"(fa1 + o), "v"(fsc + o)
                    : "memory");
            else
                asm volatile(
                    "ds_read_b128 %0, %10\n ds_read_b128 %1, %10 offset:1024\n"
                    "ds_read_u8 %2, %11\n ds_read_u8 %3, %11 offset:64\n"
                    "ds_read_b128 %4, %12\n ds_read_b128 %5, %13\n"
                    "ds_read_b128 %6, %12 offset:2048\n ds_read_b128 %7, %13 offset:2048\n"
                    "ds_read_u8 %8, %14\n ds_read_u8 %9, %14 offset:512\n"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(wa[0]), "=&v"(wa[1]), "=&v"(ws[0]), "=&v"(ws[1]), "=&v"(fa[0]), "=&v"(fb[0]),
                      "=&v"(fa[1]), "=&v"(fb[1]), "=&v"(fs[0]), "=&v"(fs[1])
                    : "v"(fw + o), "v"(fws + o), "v"(fa0 + o), "v"(fa1 + o), "v"(fsc + o)
                    : "memory");
        } else {
            ws[0] = ws[1] = 127u;
            if (ntt > 2)
                asm volatile(
                    "ds_read_b128 %0, %16\n ds_read_b128 %1, %16 offset:1024\n"
                    "ds_read_b128 %2, %16 offset:2048\n ds_read_b128 %3, %16 offset:3072\n"
                    "ds_read_b128 %4, %17\n ds_read_b128 %5, %18\n"
                    "ds_read_b128 %6, %17 offset:2048\n ds_read_b128 %7, %18 offset:2048\n"
                    "ds_read_b128 %8, %17 offset:4096\n ds_read_b128 %9, %18 offset:4096\n"
                    "ds_read_b128 %10, %17 offset:6144\n ds_read_b128 %11, %18 offset:6144\n"
                    "ds_read_u8 %12, %19\n ds_read_u8 %13, %19 offset:512\n"
                    "ds_read_u8 %14, %19 offset:32\n ds_read_u8 %15, %19 offset:544\n"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(wa[0]), "=&v"(wb[0]), "=&v"(wa[1]), "=&v"(wb[1]), "=&v"(fa[0]), "=&v"(fb[0]),
                      "=&v"(fa[1]), "=&v"(fb[1]), "=&v"(fa[2]), "=&v"(fb[2]), "=&v"(fa[3]), "=&v"(fb[3]),
                      "=&v"(fs[0]), "=&v"(fs[1]), "=&v"(fs[2]), "=&v"(fs[3])
                    : "v"(fw + o), "v"(fa0 + o), "v"(fa1 + o), "v"(fsc + o)
                    : "memory");
            else
                asm volatile(
                    "ds_read_b128 %0, %10\n ds_read_b128 %1, %10 offset:1024\n"
                    "ds_read_b128 %2, %10 offset:2048\n ds_read_b128 %3, %10 offset:3072\n"
                    "ds_read_b128 %4, %11\n ds_read_b128 %5, %12\n"
                    "ds_read_b128 %6, %11 offset:2048\n ds_read_b128 %7, %12 offset:2048\n"
                    "ds_read_u8 %8, %13\n ds_read_u8 %9, %13 offset:512\n"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(wa[0]), "=&v"(wb[0]), "=&v"(wa[1]), "=&v"(wb[1]), "=&v"(fa[0]), "=&v"(fb[0]),
                      "=&v"(fa[1]), "=&v"(fb[1]), "=&v"(fs[0]), "=&v"(fs[1])
                    : "v"(fw + o), "v"(fa0 + o), "v"(fa1 + o), "v"(fsc + o)
                    : "memory");
        }
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const i32x8_t A = {(int)wa[jt][0], (int)wa[jt][1], (int)wa[jt][2], (int)wa[jt][3],
                               (int)wb[jt][0], (int)wb[jt][1], (int)wb[jt][2], (int)wb[jt][3]};
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                if (tt >= ntt) break;
                const i32x8_t B = {(int)fa[tt][0], (int)fa[tt][1], (int)fa[tt][2], (int)fa[tt][3],
                                   (int)fb[tt][0], (int)fb[tt][1], (int)fb[tt][2], (int)fb[tt][3]};
                acc[jt][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    A, B, acc[jt][tt], WF == 0 ? 4 : 0, 0, 0, (int)ws[jt], 0, (int)fs[tt]);
            }
        }
        if (++sc < S) continue;

        // ---- the task's epilogue (its last step's slot o holds the E4M3 row scales)
        f32x4_t rs[TPW];
        if constexpr (WF == 1) {
            asm volatile("ds_read_b128 %0, %2\n ds_read_b128 %1, %2 offset:64\n s_waitcnt lgkmcnt(0)"
                         : "=&v"(rs[0]), "=&v"(rs[1])
                         : "v"(frs + o)
                         : "memory");
        } else {
            rs[0] = rs[1] = f32x4_t{1.f, 1.f, 1.f, 1.f};
        }
        if constexpr (MODE == 0) {
            // silu(gate) * up of features f0 + 4g + i, token 16 tt + t16; the
            // block of 32 features is this wave's 16 and its partner's
            // (wave ^ 1), whose maxima come through LDS
            // the exchange goes through the wave's own weight tiles of the
            // slot just read: no other wave reads them, and the slot is not
            // refilled before the next step's barrier
            const uint32_t xw = lds_l + o + (TPW * wave) * WT + 4 * t16;
            const uint32_t xr = lds_l + o + (TPW * (wave ^ 1)) * WT + 4 * t16;
            float v[4][4], bm[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
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
                bm[tt] = m;
            }
            if (g == 0)
                asm volatile(
                    "ds_write_b32 %0, %1\n ds_write_b32 %0, %2 offset:64\n"
                    "ds_write_b32 %0, %3 offset:128\n ds_write_b32 %0, %4 offset:192"
                    :
                    : "v"(xw), "v"(bm[0]), "v"(bm[1]), "v"(bm[2]), "v"(bm[3])
                    : "memory");
            barrier_lds();
            float pm[4];
            asm volatile(
                "ds_read_b32 %0, %4\n ds_read_b32 %1, %4 offset:64\n"
                "ds_read_b32 %2, %4 offset:128\n ds_read_b32 %3, %4 offset:192\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(pm[0]), "=&v"(pm[1]), "=&v"(pm[2]), "=&v"(pm[3])
                : "v"(xr)
                : "memory");
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int r = ct.c0 + 16 * tt + t16;
                const int ex = mx8_exponent(fmaxf(bm[tt], pm[tt]));
                const float inv = __builtin_amdgcn_ldexpf(1.0f, -ex);
                if (r < ct.cnt) {
                    const long arow = ct.off + r;
                    const uint32_t code = e4m3_act(v[tt][0] * inv) | (e4m3_act(v[tt][1] * inv) << 8) |
                                          (e4m3_act(v[tt][2] * inv) << 16) |
                                          (e4m3_act(v[tt][3] * inv) << 24);
                    *reinterpret_cast<uint32_t*>(a.act8 + arow * a.F + ct.f0 + 4 * g) = code;
                    if (g == 0 && (wave & 1) == 0)
                        a.act8s[arow * (a.F / 32) + ct.f0 / 32] = (uint8_t)(ex + 127);
                }
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int r = ct.c0 + 16 * tt + t16;
                if (r >= ct.cnt) continue;
#pragma unroll
                for (int j = 0; j < TPW; ++j) {
                    const f32x4_t y = acc[j][tt] * rs[j];
                    *reinterpret_cast<f32x4_t*>(a.y + (long)(ct.off + r) * a.d + ct.f0 + 16 * j + 4 * g) = y;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) acc[j][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        sc = 0;
        if (++nc < ntask) {
            ct = mx_task<MODE>(a, b + nc * G, NX, wave);
            ntt = min(4, cdiv(ct.cnt - ct.c0, 16));
        }
    }
    // the loads of steps past the end are still in flight: none may land in
    // the ring after the workgroup has left it
    DG_WAIT_VM(0);
}

// One persistent launch per product: as many workgroups as fit on the chip
// at once (LDS-bound: MXFP4 three a CU, E4M3 two), at most one per task
// there can be.
template <int MODE, int WF>
hipError_t launch_mx(const MoeArgs& a, hipStream_t st) {
    constexpr int per_cu = (160 * 1024) / mx_lds_bytes<WF>();
    static_assert(per_cu >= 1, "ring fits LDS");
    const int NX = MODE == 0 ? a.F / (32 * MX_TPW) : a.d / (64 * MX_TPW);
    const long most = (long)(cdiv(a.T * a.k, kMoeChunk) + std::min(a.E, a.T * a.k)) * NX;
    const int grid = (int)std::min<long>(most, (long)cu_count() * per_cu);
    hipLaunchKernelGGL((expert_mx_kernel<MODE, WF>), dim3(grid), dim3(256), 0, st, a, cu_count());
    return hipGetLastError();
}

}  // namespace

// the block-scaled kernels' shape limits: 128 k per step, 64 features per
// row block of the gate/up product, 128 rows of the down product
bool expert_mx_ok(const MoeArgs& a) {
    return a.F % 128 == 0 && a.d % 128 == 0 && a.u8 && a.u8s && a.act8 && a.act8s && a.order &&
           a.work &&
           (a.f4 ? (a.x_gate && a.x_up && a.x_down)
                 : (a.f8 && a.s_gate && a.s_up && a.s_down));
}

hipError_t moe_gateup_mx(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (!expert_mx_ok(a)) return hipErrorInvalidValue;
    return a.f4 ? launch_mx<0, 0>(a, st) : launch_mx<0, 1>(a, st);
}

hipError_t moe_down_mx(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (!expert_mx_ok(a)) return hipErrorInvalidValue;
    return a.f4 ? launch_mx<1, 0>(a, st) : launch_mx<1, 1>(a, st);
}

}  // namespace dg
