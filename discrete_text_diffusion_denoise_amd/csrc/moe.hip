// Mixture-of-experts half of a layer on gfx950: top-k routing, stable token
// permutation by expert, grouped SwiGLU expert GEMMs and the gated combine.
//
// Report-summary page (animattoys.com), section 2: 128 experts, the 8 best
// suited run for each token; section 5: a 256-token canvas touches many
// distinct experts, so the layer is bound by loading expert weights.  The
// grouped GEMMs therefore stream each expert's weights exactly once per
// group of 64 routed tokens, straight from HBM into MFMA operands, while the
// (small, reused) token rows come through the caches.
#include <cstdlib>

#include "common.h"
#include "kernels.h"
#include "lds_ring.h"

namespace dg {

namespace {

__device__ __forceinline__ uint32_t orderable(float z) {
    uint32_t u = __float_as_uint(z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave per token: k rounds of a wave-wide max over (logit, -index).
__global__ __launch_bounds__(256) void route_kernel(MoeArgs a) {
    const int lane = threadIdx.x & 63;
    const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const float* z = a.z + t * a.E;
    uint64_t key[4];
    float zv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        zv[i] = e < a.E ? z[e] : 0.f;
        key[i] = e < a.E ? ((uint64_t)orderable(zv[i]) << 32) | (uint32_t)(0xFFFFFFFFu - e) : 0;
    }
    float myz = 0.f;   // lane j keeps the j-th selected logit and expert
    int mye = 0;
    for (int j = 0; j < a.k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            uint32_t lo = __shfl_xor((uint32_t)best, o, 64);
            uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o, 64);
            uint64_t other = ((uint64_t)hi << 32) | lo;
            best = other > best ? other : best;
        }
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == e) key[i] = 0;
        if (lane == j) {
            myz = z[e];
            mye = e;
        }
    }
    // gates = softmax over the selected logits (selection order)
    const float z0 = __shfl(myz, 0, 64);
    const float ex = lane < a.k ? expf(myz - z0) : 0.f;
    const float s = wave_sum(ex);
    if (lane < a.k) {
        a.route[t * a.k + lane] = mye;
        a.gates[t * a.k + lane] = ex / s;
    }
}

// counts[e] = number of (token, slot) pairs routed to e.
__global__ __launch_bounds__(256) void count_kernel(MoeArgs a) {
    const int e = blockIdx.x;
    const long total = (long)a.T * a.k;
    int c = 0;
    for (long i = threadIdx.x; i < total; i += 256) c += a.route[i] == e;
    __shared__ int part[256];
    part[threadIdx.x] = c;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.counts[e] = part[0];
}

// Experts by falling count (ties: lower id) from the counts.
__global__ __launch_bounds__(256) void order_kernel(MoeArgs a) {
    const int e = threadIdx.x;
    if (e >= a.E) return;
    const int me = a.counts[e];
    int rank = 0;
    for (int e2 = 0; e2 < a.E; ++e2) {
        const int o = a.counts[e2];
        rank += (o > me) || (o == me && e2 < e);
    }
    a.order[rank] = e;
}

// One wave per expert: exclusive prefix of counts, then a stable, ordered
// placement of the pairs routed to e (ballot + popcount), so the permutation
// is deterministic.
__global__ __launch_bounds__(64) void place_kernel(MoeArgs a) {
    const int e = blockIdx.x, lane = threadIdx.x;
    int off = 0;
    for (int i = lane; i < e; i += 64) off += a.counts[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) off += __shfl_xor(off, o, 64);
    if (lane == 0) {
        a.offsets[e] = off;
        if (e == a.E - 1) a.offsets[a.E] = off + a.counts[e];
    }
    const long total = (long)a.T * a.k;
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    int run = off;
    for (long base = 0; base < total; base += 64) {
        const long i = base + lane;
        const bool match = i < total && a.route[i] == e;
        const uint64_t mask = __ballot(match);
        if (match) {
            const int slot = run + __popcll(mask & lt);
            a.perm_tok[slot] = (int32_t)(i / a.k);
            a.slot_of[i] = slot;
        }
        run += __popcll(mask);
    }
}

// Grouped expert GEMMs, weight streaming.  A workgroup owns a block of weight
// rows of one expert -- MODE 0: 32 rows of W_gate and the same 32 rows of
// W_up (SwiGLU epilogue into act); MODE 1: 32 rows of W_down (fp32 out) --
// and walks K in 64-wide stages.  Each stage's weight rows are read as full
// 128-byte row segments (8 threads per row, coalesced), two stages ahead of
// use through registers, and staged in LDS together with the stage's token
// rows (gathered through the permutation for MODE 0).  Waves: column tile
// ct = w & 1 (16 rows each), token tiles {w >> 1, (w >> 1) + 2} of the
// 64-token group.  Token groups beyond 64 re-read the block's weights (L2).
constexpr int XK = 64;             // k per stage
constexpr int XROW = XK + 8;       // LDS row stride (elements)
constexpr int XG = 64;             // tokens per group

template <typename T, int MODE>
__global__ __launch_bounds__(256) void expert_kernel(MoeArgs a) {
    if (a.halt && *a.halt) return;
    constexpr int RW = MODE == 0 ? 64 : 32;           // weight rows in LDS
    constexpr int CE = 16 / (int)sizeof(T);           // elements per 16-byte chunk
    constexpr int CPR = XK / CE;                      // chunks per row per stage
    constexpr int WCH = RW * CPR / 256;               // weight chunks per thread
    constexpr int XCH = XG * CPR / 256;               // token chunks per thread
    __shared__ __align__(16) T Ws[2][RW * XROW];
    __shared__ __align__(16) T Xs[2][XG * XROW];

    const int e = blockIdx.y;
    const int off = a.offsets[e], cnt = a.offsets[e + 1] - off;
    if (cnt == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int ct = wave & 1, mp = wave >> 1;
    const int K = MODE == 0 ? a.d : a.F;
    const int NOUT = MODE == 0 ? a.F : a.d;            // output columns of this expert
    const int c0 = blockIdx.x * 32;                    // first output column of the block
    const T* Wg = reinterpret_cast<const T*>(MODE == 0 ? a.w_gate : a.w_down);
    const T* Wu = reinterpret_cast<const T*>(a.w_up);
    const T* X = reinterpret_cast<const T*>(MODE == 0 ? a.u : a.act);
    const int nst = cdiv(K, XK);
    // blocks start their K walk at different stages so concurrent blocks read
    // different offsets within their weight rows
    const int rot = a.k_rotate ? (int)((blockIdx.x + (long)blockIdx.y * 5) % nst) : 0;

    // this thread's weight chunks: (row, k chunk) -> global row pointer
    const T* wsrc[WCH];
    int wrow[WCH], wkc[WCH];
    bool wval[WCH];
#pragma unroll
    for (int c = 0; c < WCH; ++c) {
        const int ch = tid + c * 256;
        wrow[c] = ch / CPR;
        wkc[c] = (ch % CPR) * CE;
        const int r = wrow[c] % 32;                     // row within the gate / up half
        const int col = c0 + r;
        wval[c] = col < NOUT;
        const T* base = (MODE == 0 && wrow[c] >= 32) ? Wu : Wg;
        wsrc[c] = base + ((long)e * NOUT + (wval[c] ? col : 0)) * K;
    }

    for (int mg = 0; mg < cnt; mg += XG) {
        // this thread's token chunks for the group
        const T* xsrc[XCH];
        int xrow[XCH], xkc[XCH];
        bool xval[XCH];
#pragma unroll
        for (int c = 0; c < XCH; ++c) {
            const int ch = tid + c * 256;
            xrow[c] = ch / CPR;
            xkc[c] = (ch % CPR) * CE;
            xval[c] = mg + xrow[c] < cnt;
            long src = 0;
            if (xval[c]) src = MODE == 0 ? (long)a.perm_tok[off + mg + xrow[c]] : (long)(off + mg + xrow[c]);
            xsrc[c] = X + src * K;
        }
        f32x4_t ag[2], au[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            ag[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            au[q] = ag[q];
        }
        uint4 wA[WCH], xA[XCH], wB[WCH], xB[XCH];

#define DG_XLOAD(ST, WR, XR)                                                                  \
        {                                                                                     \
            int sr_ = (ST) + rot;                                                             \
            if (sr_ >= nst) sr_ -= nst;                                                       \
            const int kb_ = sr_ * XK;                                                         \
            _Pragma("unroll") for (int c = 0; c < WCH; ++c) {                                 \
                const int k_ = kb_ + wkc[c];                                                  \
                WR[c] = (wval[c] && k_ < K) ? *reinterpret_cast<const uint4*>(wsrc[c] + k_)   \
                                            : make_uint4(0, 0, 0, 0);                         \
            }                                                                                 \
            _Pragma("unroll") for (int c = 0; c < XCH; ++c) {                                 \
                const int k_ = kb_ + xkc[c];                                                  \
                XR[c] = (xval[c] && k_ < K) ? *reinterpret_cast<const uint4*>(xsrc[c] + k_)   \
                                            : make_uint4(0, 0, 0, 0);                         \
            }                                                                                 \
        }
#define DG_XSTORE(BUF, WR, XR)                                                                \
        {                                                                                     \
            _Pragma("unroll") for (int c = 0; c < WCH; ++c)                                   \
                *reinterpret_cast<uint4*>(&Ws[BUF][wrow[c] * XROW + wkc[c]]) = WR[c];         \
            _Pragma("unroll") for (int c = 0; c < XCH; ++c)                                   \
                *reinterpret_cast<uint4*>(&Xs[BUF][xrow[c] * XROW + xkc[c]]) = XR[c];         \
        }
#define DG_XCOMPUTE(BUF)                                                                      \
        _Pragma("unroll") for (int s_ = 0; s_ < XK / 32; ++s_) {                              \
            Frag<T> fg, fu;                                                                   \
            load_frag(fg, &Ws[BUF][(ct * 16 + r16) * XROW + s_ * 32 + g4 * 8]);               \
            if (MODE == 0) load_frag(fu, &Ws[BUF][(32 + ct * 16 + r16) * XROW + s_ * 32 + g4 * 8]); \
            _Pragma("unroll") for (int q = 0; q < 2; ++q) {                                   \
                const int mt = mp + 2 * q;                                                    \
                if (mg + 16 * mt < cnt) {                                                     \
                    Frag<T> fx;                                                               \
                    load_frag(fx, &Xs[BUF][(16 * mt + r16) * XROW + s_ * 32 + g4 * 8]);       \
                    mma(ag[q], fx, fg);                                                       \
                    if (MODE == 0) mma(au[q], fx, fu);                                        \
                }                                                                             \
            }                                                                                 \
        }

        DG_XLOAD(0, wA, xA)
        DG_XSTORE(0, wA, xA)
        if (nst > 1) DG_XLOAD(1, wB, xB)
        if (nst > 2) DG_XLOAD(2, wA, xA)
        __syncthreads();
        // stage st: LDS buffer st & 1; register set of stage st+1 is stored at
        // the end of the iteration, stage st+2 is in flight in the other set
        for (int st = 0; st < nst; st += 2) {
            DG_XCOMPUTE(0)
            if (st + 1 < nst) DG_XSTORE(1, wB, xB)
            __syncthreads();
            if (st + 3 < nst) DG_XLOAD(st + 3, wB, xB)
            if (st + 1 >= nst) break;
            DG_XCOMPUTE(1)
            if (st + 2 < nst) DG_XSTORE(0, wA, xA)
            __syncthreads();
            if (st + 4 < nst) DG_XLOAD(st + 4, wA, xA)
        }
#undef DG_XLOAD
#undef DG_XSTORE
#undef DG_XCOMPUTE

        // lane holds tokens 4*g4 + i of tile mt, output column c0 + ct*16 + r16
        const int col = c0 + ct * 16 + r16;
        if (col < NOUT) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int mt = mp + 2 * q;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = mg + 16 * mt + 4 * g4 + i;
                    if (row >= cnt) continue;
                    if constexpr (MODE == 0) {
                        const float gv = ag[q][i], uv = au[q][i];
                        const float sv = gv / (1.0f + __expf(-gv));
                        reinterpret_cast<T*>(a.act)[(long)(off + row) * a.F + col] =
                            Elt<T>::from_f(sv * uv);
                    } else {
                        a.y[(long)(off + row) * a.d + col] = ag[q][i];
                    }
                }
            }
        }
        __syncthreads();   // LDS reuse by the next token group
    }
}

// bf16 expert GEMMs with direct-to-LDS loads.  Same work split and epilogue
// as expert_kernel, but weight and token rows go from memory straight into
// a ring of four LDS stages (64-wide k) with global_load_lds, three stages in
// flight while one is multiplied, so the weight stream is not throttled by
// register staging.  Rows are 128 bytes per stage; chunk c of row r sits in
// slot c ^ (r & 7), which keeps the fragment reads free of bank conflicts.
// Fragment reads are one asm block per stage ending in its own
// lgkmcnt(0) (the ring order already guarantees their loads have landed).

// One expert's token groups against one block of weight rows: a four-stage
// ring of direct-to-LDS loads (8 KiB of weight rows x 64 k and 32 * G token
// rows x 64 k per stage), G = 1 or 2 groups of 32 tokens per pass over the
// weights.  bf16 weights: 64 rows (two halves of 32 columns) per block.
// F8: 128 rows of E4M3 codes (two halves of 64 columns; 64 bytes per row and
// stage), widened to bf16 in registers (exactly: E4M3 values are bf16
// values) and scaled per output column after the sum.
struct XdCtx {
    int e, off, cnt, K, NOUT, c0, n, rot;
    int lane, wave, r16, g4, ct, mp, lr, lc;
    const char* wsrc[2];     // byte addresses of this lane's weight chunks at k = 0
    const bf16_t* X;
    const uint8_t* ssrc;     // MXFP4: this lane's 16 scale bytes of stage 0
    long sstride;            // MXFP4: scale bytes from one stage to the next
};

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// 8 E4M3 codes (two words, increasing k) -> 8 bf16 values
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    return u32x4{pack_bf2(a.x, a.y), pack_bf2(b.x, b.y), pack_bf2(c.x, c.y), pack_bf2(d.x, d.y)};
}

// 8 E2M1 codes (a word, the even k in the low nibble of each byte) times a
// power-of-two scale -> 8 bf16 values, exact (every such product is a bf16
// value): gfx950 converts the two codes of a selected byte per instruction,
// low nibble first (checked on all 256 bytes and several scales)
__device__ __forceinline__ u32x4 e2m1x8_to_bf16(uint32_t w, float scale) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3))};
}

// FMT: 0 bf16 weights, 1 E4M3 codes with per-row scales, 2 MXFP4 (E2M1 codes,
// an E8M0 scale per 32 k)
template <int MODE, int G, int FMT>
__device__ __forceinline__ void expert_groups(const MoeArgs& a, const XdCtx& c, unsigned char* w0,
                                              unsigned char* w1, unsigned char* w2, unsigned char* w3,
                                              unsigned char* x0, unsigned char* x1, unsigned char* x2,
                                              unsigned char* x3, unsigned char* s0, unsigned char* s1,
                                              unsigned char* s2, unsigned char* s3) {
    constexpr bool F8 = FMT == 1, F4 = FMT == 2;
    constexpr int WQ = 2;                              // weight DMAs per wave per stage
    constexpr int SQ = F4 ? 1 : 0;                     // scale DMAs per wave per stage
    constexpr int PER = WQ + G + SQ;                   // DMAs per wave per stage
    constexpr int WSTAGE = F4 ? 32 : (F8 ? 64 : 128);  // weight bytes per row and stage
    constexpr int J = F4 ? 4 : (F8 ? 2 : 1);           // 16-column tiles per half and wave
    constexpr int HALF = 32 * J;                       // columns per half of the block
    const int n = c.n, rot = c.rot, mp = c.mp, ct = c.ct, r16 = c.r16, g4 = c.g4;
    const int wblk = c.wave * WQ * 1024;
    const int xblk = c.wave * G * 1024;
    const int roff = r16 * 128;
    // output columns of the lane (tile ct + 2j of the first half; the
    // second half is the up projection, or the down columns HALF later)
    // and, for 8-bit weights, their scales
    int col[J];
    float sc0[J], sc1[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        col[j] = c.c0 + (ct + 2 * j) * 16 + r16;
        sc0[j] = 1.0f;
        sc1[j] = 1.0f;
        if (F8 && col[j] < c.NOUT) {
            if (MODE == 0) {
                sc0[j] = a.s_gate[(long)c.e * c.NOUT + col[j]];
                sc1[j] = a.s_up[(long)c.e * c.NOUT + col[j]];
            } else {
                sc0[j] = a.s_down[(long)c.e * c.NOUT + col[j]];
                sc1[j] = col[j] + HALF < c.NOUT ? a.s_down[(long)c.e * c.NOUT + col[j] + HALF] : 1.0f;
            }
        }
    }
    for (int mg = 0; mg < c.cnt; mg += 32 * G) {
        const bf16_t* xsrc[G];
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const int tok = min(mg + (c.wave * G + q) * 8 + c.lr, c.cnt - 1);
            const long src = MODE == 0 ? (long)a.perm_tok[c.off + tok] : (long)(c.off + tok);
            xsrc[q] = c.X + src * c.K + c.lc;
        }
        // wave: token tiles mp (and mp + 2 when G = 2), column tiles ct + 2j
        // of both halves of the weight block
        f32x4_t ag[G][J], au[G][J];
        bool tv[G];
#pragma unroll
        for (int q = 0; q < G; ++q) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                ag[q][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                au[q][j] = ag[q][j];
            }
            tv[q] = mg + 16 * (mp + 2 * q) < c.cnt;
        }

#define XD_ISSUE(ST, WB, XB, SB)                                                                  \
        {                                                                                         \
            int sr_ = (ST) + rot;                                                                 \
            if (sr_ >= n) sr_ -= n;                                                               \
            const int k_ = sr_ * 64;                                                              \
            _Pragma("unroll") for (int q = 0; q < WQ; ++q)                                        \
                __builtin_amdgcn_global_load_lds((glb_void*)(c.wsrc[q] + (long)sr_ * WSTAGE),     \
                                                 (lds_void*)((WB) + wblk + q * 1024), 16, 0, 0);  \
            _Pragma("unroll") for (int q = 0; q < G; ++q)                                         \
                __builtin_amdgcn_global_load_lds((glb_void*)(xsrc[q] + k_),                       \
                                                 (lds_void*)((XB) + xblk + q * 1024), 16, 0, 0);  \
            if (F4 && c.lane < 8)                                                                 \
                __builtin_amdgcn_global_load_lds((glb_void*)(c.ssrc + (long)sr_ * c.sstride),     \
                                                 (lds_void*)((SB) + c.wave * 128), 16, 0, 0);     \
        }
        // fragments: token rows 16*(mp + 2q) + r16; weight rows (ct + 2j)*16
        // + r16 of each half.  bf16 weights: k-step s of a lane is chunk
        // 4*s + g4 of both operands; 8-bit weights: the lane's 16 codes are
        // chunk g4 of the 64-byte row (k 16*g4 .. 16*g4+15), so its token
        // chunks are 2*g4 (k-step 0) and 2*g4 + 1 (k-step 1): every k of the
        // stage is in exactly one k-step of one lane group, as the sum needs
#define XD_COMPUTE(WB, XB, SB)                                                                    \
        {                                                                                         \
            u32x4 fga[J], fgb[J], fua[J], fub[J], fxa[G], fxb[G];                                 \
            const uint32_t xa = lds_addr(XB) + (16 * mp) * 128 + roff;                            \
            const int xs = r16 & 7;                                                               \
            const uint32_t sa = (F8 || F4) ? ((2 * g4) ^ xs) << 4 : (g4 ^ xs) << 4;               \
            const uint32_t sb = (F8 || F4) ? ((2 * g4 + 1) ^ xs) << 4 : ((4 + g4) ^ xs) << 4;     \
            if (F4) {                                                                             \
                /* weight row (ct + 2j)*16 + r16 of each half (32 bytes a row,  */                \
                /* 16-byte chunk c in slot c ^ bit 3 of the row): the lane's 8  */                \
                /* bytes are codes k 16*g4 .. 16*g4+15 of the stage, one MX     */                \
                /* block, whose scale byte sits at half*256 + row*2 + g4/2      */                \
                const int wr0 = ct * 16 + r16;                                                    \
                const uint32_t wq_ = lds_addr(WB) + wr0 * 32 +                                    \
                                     ((((g4 >> 1) ^ ((r16 >> 3) & 1))) << 4) + ((g4 & 1) << 3);   \
                const uint32_t sq_ = lds_addr(SB) + wr0 * 2 + (g4 >> 1);                          \
                uint2 cw[2 * J];                                                                  \
                uint32_t cs[2 * J];                                                               \
                if (G == 1) {                                                                     \
                    asm volatile(                                                                 \
                        "ds_read_b128 %0, %18\n ds_read_b128 %1, %19\n"                            \
                        "ds_read_b64 %2, %20 offset:0\n ds_read_b64 %3, %20 offset:1024\n"        \
                        "ds_read_b64 %4, %20 offset:2048\n ds_read_b64 %5, %20 offset:3072\n"     \
                        "ds_read_b64 %6, %20 offset:4096\n ds_read_b64 %7, %20 offset:5120\n"     \
                        "ds_read_b64 %8, %20 offset:6144\n ds_read_b64 %9, %20 offset:7168\n"     \
                        "ds_read_u8 %10, %21 offset:0\n ds_read_u8 %11, %21 offset:64\n"          \
                        "ds_read_u8 %12, %21 offset:128\n ds_read_u8 %13, %21 offset:192\n"       \
                        "ds_read_u8 %14, %21 offset:256\n ds_read_u8 %15, %21 offset:320\n"       \
                        "ds_read_u8 %16, %21 offset:384\n ds_read_u8 %17, %21 offset:448\n"       \
                        "s_waitcnt lgkmcnt(0)"                                                     \
                        : "=&v"(fxa[0]), "=&v"(fxb[0]), "=&v"(cw[0]), "=&v"(cw[1]), "=&v"(cw[2]),   \
                          "=&v"(cw[3]), "=&v"(cw[4]), "=&v"(cw[5]), "=&v"(cw[6]), "=&v"(cw[7]),     \
                          "=&v"(cs[0]), "=&v"(cs[1]), "=&v"(cs[2]), "=&v"(cs[3]), "=&v"(cs[4]),     \
                          "=&v"(cs[5]), "=&v"(cs[6]), "=&v"(cs[7])                                \
                        : "v"(xa + sa), "v"(xa + sb), "v"(wq_), "v"(sq_)                          \
                        : "memory");                                                              \
                } else {                                                                          \
                    asm volatile(                                                                 \
                        "ds_read_b128 %0, %20\n ds_read_b128 %1, %21\n"                            \
                        "ds_read_b128 %2, %20 offset:4096\n ds_read_b128 %3, %21 offset:4096\n"   \
                        "ds_read_b64 %4, %22 offset:0\n ds_read_b64 %5, %22 offset:1024\n"        \
                        "ds_read_b64 %6, %22 offset:2048\n ds_read_b64 %7, %22 offset:3072\n"     \
                        "ds_read_b64 %8, %22 offset:4096\n ds_read_b64 %9, %22 offset:5120\n"     \
                        "ds_read_b64 %10, %22 offset:6144\n ds_read_b64 %11, %22 offset:7168\n"   \
                        "ds_read_u8 %12, %23 offset:0\n ds_read_u8 %13, %23 offset:64\n"          \
                        "ds_read_u8 %14, %23 offset:128\n ds_read_u8 %15, %23 offset:192\n"       \
                        "ds_read_u8 %16, %23 offset:256\n ds_read_u8 %17, %23 offset:320\n"       \
                        "ds_read_u8 %18, %23 offset:384\n ds_read_u8 %19, %23 offset:448\n"       \
                        "s_waitcnt lgkmcnt(0)"                                                     \
                        : "=&v"(fxa[0]), "=&v"(fxb[0]), "=&v"(fxa[G - 1]), "=&v"(fxb[G - 1]),      \
                          "=&v"(cw[0]), "=&v"(cw[1]), "=&v"(cw[2]), "=&v"(cw[3]), "=&v"(cw[4]),     \
                          "=&v"(cw[5]), "=&v"(cw[6]), "=&v"(cw[7]), "=&v"(cs[0]), "=&v"(cs[1]),     \
                          "=&v"(cs[2]), "=&v"(cs[3]), "=&v"(cs[4]), "=&v"(cs[5]), "=&v"(cs[6]),     \
                          "=&v"(cs[7])                                                            \
                        : "v"(xa + sa), "v"(xa + sb), "v"(wq_), "v"(sq_)                          \
                        : "memory");                                                              \
                }                                                                                 \
                _Pragma("unroll") for (int j = 0; j < J; ++j) {                                   \
                    const float fg_ = __builtin_amdgcn_ldexpf(1.0f, (int)cs[j] - 127);            \
                    const float fu_ = __builtin_amdgcn_ldexpf(1.0f, (int)cs[J + j] - 127);        \
                    fga[j] = e2m1x8_to_bf16(cw[j].x, fg_);                                        \
                    fgb[j] = e2m1x8_to_bf16(cw[j].y, fg_);                                        \
                    fua[j] = e2m1x8_to_bf16(cw[J + j].x, fu_);                                    \
                    fub[j] = e2m1x8_to_bf16(cw[J + j].y, fu_);                                    \
                }                                                                                 \
            } else if (F8) {                                                                             \
                const int wr0 = ct * 16 + r16, wr1 = wr0 + 32;                                    \
                const uint32_t wb_ = lds_addr(WB);                                                \
                const uint32_t g0_ = wb_ + wr0 * 64 + ((g4 ^ swz(wr0)) << 4);                    \
                const uint32_t g1_ = wb_ + wr1 * 64 + ((g4 ^ swz(wr1)) << 4);                    \
                const uint32_t u0_ = wb_ + (wr0 + 64) * 64 + ((g4 ^ swz(wr0 + 64)) << 4);        \
                const uint32_t u1_ = wb_ + (wr1 + 64) * 64 + ((g4 ^ swz(wr1 + 64)) << 4);        \
                u32x4 cg0, cg1, cu0, cu1;                                                         \
                if (G == 1) {                                                                     \
                    asm volatile(                                                                 \
                        "ds_read_b128 %0, %6\n ds_read_b128 %1, %7\n"                              \
                        "ds_read_b128 %2, %8\n ds_read_b128 %3, %9\n"                              \
                        "ds_read_b128 %4, %10\n ds_read_b128 %5, %11\n"                            \
                        "s_waitcnt lgkmcnt(0)"                                                     \
                        : "=&v"(fxa[0]), "=&v"(fxb[0]), "=&v"(cg0), "=&v"(cg1), "=&v"(cu0), "=&v"(cu1) \
                        : "v"(xa + sa), "v"(xa + sb), "v"(g0_), "v"(g1_), "v"(u0_), "v"(u1_)      \
                        : "memory");                                                              \
                } else {                                                                          \
                    asm volatile(                                                                 \
                        "ds_read_b128 %0, %8\n ds_read_b128 %1, %9\n"                              \
                        "ds_read_b128 %2, %10\n ds_read_b128 %3, %11\n"                            \
                        "ds_read_b128 %4, %12\n ds_read_b128 %5, %13\n"                            \
                        "ds_read_b128 %6, %14\n ds_read_b128 %7, %15\n"                            \
                        "s_waitcnt lgkmcnt(0)"                                                     \
                        : "=&v"(fxa[0]), "=&v"(fxb[0]), "=&v"(fxa[G - 1]), "=&v"(fxb[G - 1]),      \
                          "=&v"(cg0), "=&v"(cg1), "=&v"(cu0), "=&v"(cu1)                          \
                        : "v"(xa + sa), "v"(xa + sb), "v"(xa + 32 * 128 + sa),                    \
                          "v"(xa + 32 * 128 + sb), "v"(g0_), "v"(g1_), "v"(u0_), "v"(u1_)         \
                        : "memory");                                                              \
                }                                                                                 \
                fga[0] = e4m3x8_to_bf16(cg0[0], cg0[1]);                                          \
                fgb[0] = e4m3x8_to_bf16(cg0[2], cg0[3]);                                          \
                fua[0] = e4m3x8_to_bf16(cu0[0], cu0[1]);                                          \
                fub[0] = e4m3x8_to_bf16(cu0[2], cu0[3]);                                          \
                fga[J - 1] = e4m3x8_to_bf16(cg1[0], cg1[1]);                                      \
                fgb[J - 1] = e4m3x8_to_bf16(cg1[2], cg1[3]);                                      \
                fua[J - 1] = e4m3x8_to_bf16(cu1[0], cu1[1]);                                      \
                fub[J - 1] = e4m3x8_to_bf16(cu1[2], cu1[3]);                                      \
            } else {                                                                              \
                const uint32_t wa = lds_addr(WB) + (ct * 16) * 128 + roff;                        \
                if (G == 1) {                                                                     \
                    asm volatile(                                                                 \
                        "ds_read_b128 %0, %6\n ds_read_b128 %1, %7\n"                              \
                        "ds_read_b128 %2, %8\n ds_read_b128 %3, %9\n"                              \
                        "ds_read_b128 %4, %10\n ds_read_b128 %5, %11\n"                            \
                        "s_waitcnt lgkmcnt(0)"                                                     \
                        : "=&v"(fxa[0]), "=&v"(fxb[0]), "=&v"(fga[0]), "=&v"(fgb[0]), "=&v"(fua[0]), \
                          "=&v"(fub[0])                                                           \
                        : "v"(xa + sa), "v"(xa + sb), "v"(wa + sa), "v"(wa + sb), "v"(wa + 32 * 128 + sa), \
                          "v"(wa + 32 * 128 + sb)                                                 \
                        : "memory");                                                              \
                } else {                                                                          \
                    asm volatile(                                                                 \
                        "ds_read_b128 %0, %8\n ds_read_b128 %1, %9\n"                              \
                        "ds_read_b128 %2, %10\n ds_read_b128 %3, %11\n"                            \
                        "ds_read_b128 %4, %12\n ds_read_b128 %5, %13\n"                            \
                        "ds_read_b128 %6, %14\n ds_read_b128 %7, %15\n"                            \
                        "s_waitcnt lgkmcnt(0)"                                                     \
                        : "=&v"(fxa[0]), "=&v"(fxb[0]), "=&v"(fxa[G - 1]), "=&v"(fxb[G - 1]),      \
                          "=&v"(fga[0]), "=&v"(fgb[0]), "=&v"(fua[0]), "=&v"(fub[0])              \
                        : "v"(xa + sa), "v"(xa + sb), "v"(xa + 32 * 128 + sa), "v"(xa + 32 * 128 + sb), \
                          "v"(wa + sa), "v"(wa + sb), "v"(wa + 32 * 128 + sa), "v"(wa + 32 * 128 + sb) \
                        : "memory");                                                              \
                }                                                                                 \
            }                                                                                     \
            _Pragma("unroll") for (int q = 0; q < G; ++q) {                                       \
                if (tv[q]) {                                                                      \
                    _Pragma("unroll") for (int j = 0; j < J; ++j) {                               \
                        ag[q][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                       \
                            __builtin_bit_cast(bf16x8_t, fxa[q]), __builtin_bit_cast(bf16x8_t, fga[j]), ag[q][j], 0, 0, 0); \
                        ag[q][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                       \
                            __builtin_bit_cast(bf16x8_t, fxb[q]), __builtin_bit_cast(bf16x8_t, fgb[j]), ag[q][j], 0, 0, 0); \
                        au[q][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                       \
                            __builtin_bit_cast(bf16x8_t, fxa[q]), __builtin_bit_cast(bf16x8_t, fua[j]), au[q][j], 0, 0, 0); \
                        au[q][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                       \
                            __builtin_bit_cast(bf16x8_t, fxb[q]), __builtin_bit_cast(bf16x8_t, fub[j]), au[q][j], 0, 0, 0); \
                    }                                                                             \
                }                                                                                 \
            }                                                                                     \
        }
#define XD_STAGE(t, CW, CX, CS, NW, NX, NS)                  \
        {                                                    \
            if ((t) + 2 < n)                                 \
                DG_WAIT_VM(2 * PER);                         \
            else if ((t) + 1 < n)                            \
                DG_WAIT_VM(PER);                             \
            else                                             \
                DG_WAIT_VM(0);                               \
            barrier_lds();                                   \
            if ((t) + 3 < n) XD_ISSUE((t) + 3, NW, NX, NS);  \
            XD_COMPUTE(CW, CX, CS);                          \
        }
        XD_ISSUE(0, w0, x0, s0);
        XD_ISSUE(1, w1, x1, s1);
        XD_ISSUE(2, w2, x2, s2);
        for (int t = 0; t < n; t += 4) {
            XD_STAGE(t, w0, x0, s0, w3, x3, s3);
            XD_STAGE(t + 1, w1, x1, s1, w0, x0, s0);
            XD_STAGE(t + 2, w2, x2, s2, w1, x1, s1);
            XD_STAGE(t + 3, w3, x3, s3, w2, x2, s2);
        }
#undef XD_STAGE
#undef XD_COMPUTE
#undef XD_ISSUE

        // lane holds tokens 4*g4 + i of tile mp + 2q, output columns col[j]
        // (and col[j] + HALF for the second half of the down projection)
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if (col[j] >= c.NOUT) continue;
#pragma unroll
            for (int q = 0; q < G; ++q) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = mg + 16 * (mp + 2 * q) + 4 * g4 + i;
                    if (row >= c.cnt) continue;
                    if constexpr (MODE == 0) {
                        const float gv = F8 ? ag[q][j][i] * sc0[j] : ag[q][j][i];
                        const float uv = F8 ? au[q][j][i] * sc1[j] : au[q][j][i];
                        const float sv = gv / (1.0f + __expf(-gv));
                        reinterpret_cast<bf16_t*>(a.act)[(long)(c.off + row) * a.F + col[j]] =
                            f2bf(sv * uv);
                    } else {
                        a.y[(long)(c.off + row) * a.d + col[j]] = F8 ? ag[q][j][i] * sc0[j] : ag[q][j][i];
                        if (col[j] + HALF < c.NOUT)
                            a.y[(long)(c.off + row) * a.d + col[j] + HALF] =
                                F8 ? au[q][j][i] * sc1[j] : au[q][j][i];
                    }
                }
            }
        }
        // the next group's loads refill the ring only after every wave is done
        barrier_lds();
    }
}

// Blocks of weight rows (bf16: 64 rows = gate and up rows of 32 columns
// (MODE 0) or 64 columns of the down projection (MODE 1); 8-bit: 128 rows,
// twice the columns); blockIdx.y walks the experts in `order` when it is
// set.  An expert with at most 32 tokens (most of them: a 256-token canvas
// makes 2048 assignments over 128 experts) runs groups of 32, a busier one
// groups of 64, so its weights are streamed fewer times.
template <int MODE, int FMT>
__global__ __launch_bounds__(256) void expert_dma_kernel(MoeArgs a) {
    if (a.halt && *a.halt) return;
    constexpr bool F8 = FMT == 1, F4 = FMT == 2;
    __shared__ __align__(1024) unsigned char w0[64 * 128], x0[8192];
    __shared__ __align__(1024) unsigned char w1[64 * 128], x1[8192];
    __shared__ __align__(1024) unsigned char w2[64 * 128], x2[8192];
    __shared__ __align__(1024) unsigned char w3[64 * 128], x3[8192];
    // MXFP4 scale bytes of a stage: 256 rows x 2 blocks
    __shared__ __align__(16) unsigned char s0[F4 ? 512 : 16], s1[F4 ? 512 : 16];
    __shared__ __align__(16) unsigned char s2[F4 ? 512 : 16], s3[F4 ? 512 : 16];
    constexpr int HALF = F4 ? 128 : (F8 ? 64 : 32);    // columns per half of a block

    XdCtx c;
    // the busiest experts first, so their longer blocks do not form the tail
    c.e = a.order ? a.order[blockIdx.y] : (int)blockIdx.y;
    c.off = a.offsets[c.e];
    c.cnt = a.offsets[c.e + 1] - c.off;
    if (c.cnt == 0) return;
    const int tid = threadIdx.x;
    c.lane = tid & 63;
    c.wave = tid >> 6;
    c.r16 = c.lane & 15;
    c.g4 = c.lane >> 4;
    c.ct = c.wave & 1;
    c.mp = c.wave >> 1;
    c.K = MODE == 0 ? a.d : a.F;
    c.NOUT = MODE == 0 ? a.F : a.d;
    c.c0 = blockIdx.x * (MODE == 0 ? HALF : 2 * HALF);
    c.n = __builtin_amdgcn_readfirstlane(c.K / 64);   // stages, a multiple of 4
    // the starting stage depends on (column block, expert) only, so a token's
    // sum runs in the same order whatever the other tokens of the batch are
    c.rot = __builtin_amdgcn_readfirstlane(a.k_rotate ? (int)((blockIdx.x + c.e * 5) % c.n) : 0);
    const char* Wg = reinterpret_cast<const char*>(MODE == 0 ? a.w_gate : a.w_down);
    const char* Wu = reinterpret_cast<const char*>(a.w_up);
    c.X = reinterpret_cast<const bf16_t*>(MODE == 0 ? a.u : a.act);
    // token DMA lanes: an instruction fills 8 rows x 128 bytes; lane l takes
    // row l / 8 of them and global chunk (l % 8) ^ (row & 7)
    c.lr = c.lane >> 3;
    c.lc = ((c.lane & 7) ^ c.lr) * 8;                 // element offset (rows are 8-aligned)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (F4) {
            // weight DMA lanes: an instruction fills 32 rows x 32 bytes; lane
            // l takes row l / 2 and global chunk (l % 2) ^ (bit 3 of the row)
            const int r = (c.wave * 2 + q) * 32 + (c.lane >> 1);   // row within the block
            const int rr = MODE == 0 ? (r & (HALF - 1)) : r;
            const int col = min(c.c0 + rr, c.NOUT - 1);
            const char* base = (MODE == 0 && r >= HALF) ? Wu : Wg;
            c.wsrc[q] = base + ((long)c.e * c.NOUT + col) * (c.K / 2) +
                        (((c.lane & 1) ^ ((r >> 3) & 1)) << 4);
        } else if (F8) {
            // weight DMA lanes: an instruction fills 16 rows x 64 bytes; lane l
            // takes row l / 4 and global chunk (l % 4) ^ swz(row)
            const int r = (c.wave * 2 + q) * 16 + (c.lane >> 2);   // row within the block
            const int rr = MODE == 0 ? (r & (HALF - 1)) : r;
            const int col = min(c.c0 + rr, c.NOUT - 1);
            const char* base = (MODE == 0 && r >= HALF) ? Wu : Wg;
            c.wsrc[q] = base + ((long)c.e * c.NOUT + col) * c.K + (((c.lane & 3) ^ swz(r)) << 4);
        } else {
            const int r = (c.wave * 2 + q) * 8 + c.lr;             // row within the block
            const int rr = MODE == 0 ? (r & (HALF - 1)) : r;
            const int col = min(c.c0 + rr, c.NOUT - 1);
            const char* base = (MODE == 0 && r >= HALF) ? Wu : Wg;
            c.wsrc[q] = base + (((long)c.e * c.NOUT + col) * c.K + c.lc) * 2;
        }
    }
    c.ssrc = nullptr;
    c.sstride = 0;
    if (F4) {
        // scale DMA lanes 0..7 of wave w: bytes [128 w, 128 w + 128) of the
        // stage's 512 (gate rows c0.. then up rows c0.., or down rows c0..)
        const uint8_t* X = MODE == 0 ? (c.wave < 2 ? a.x_gate : a.x_up) : a.x_down;
        const int piece = MODE == 0 ? (c.wave & 1) : c.wave;
        c.ssrc = X + ((long)c.e * c.NOUT + c.c0) * 2 + piece * 128 + (c.lane & 7) * 16;
        c.sstride = (long)a.E * c.NOUT * 2;
    }
    if (__builtin_amdgcn_readfirstlane(c.cnt) <= 32)
        expert_groups<MODE, 1, FMT>(a, c, w0, w1, w2, w3, x0, x1, x2, x3, s0, s1, s2, s3);
    else
        expert_groups<MODE, 2, FMT>(a, c, w0, w1, w2, w3, x0, x1, x2, x3, s0, s1, s2, s3);
}

// Counts, offsets and the stable placement in one workgroup.  The
// assignments are cut into PW contiguous ranges, one per wave: per-range
// expert counts (LDS atomics), an exclusive prefix over (expert, range),
// then each wave walks its range 64 assignments at a time.  Lanes holding
// the same expert find each other by ballots over the expert's bits; a
// lane's slot is its range's running offset for the expert plus the number
// of lower lanes in its group, and the group's highest lane advances the
// offset.  Same permutation as the per-expert scan (assignments of an
// expert in increasing order).
constexpr int PW = 16;             // waves of the placement workgroup

__global__ __launch_bounds__(64 * PW) void place_all_kernel(MoeArgs a) {
    __shared__ int cw[PW][256];    // per-range counts, then per-range running offsets
    __shared__ int tot[256];       // per-expert totals, then expert offsets
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int total = a.T * a.k;
    const int per = cdiv(cdiv(total, 64), PW) * 64;    // assignments per range
    const int i0 = min(total, wave * per), i1 = min(total, (wave + 1) * per);
    for (int x = tid; x < PW * 256; x += 64 * PW) (&cw[0][0])[x] = 0;
    __syncthreads();
    for (int i = i0 + lane; i < i1; i += 64) atomicAdd(&cw[wave][a.route[i]], 1);
    __syncthreads();
    if (tid < 256) {
        int c = 0;
        for (int w = 0; w < PW; ++w) c += cw[w][tid];
        tot[tid] = c;
    }
    __syncthreads();
    if (a.order && tid < a.E) {                        // rank by falling count
        const int me = tot[tid];
        int rank = 0;
        for (int e2 = 0; e2 < a.E; ++e2) {
            const int o = tot[e2];
            rank += (o > me) || (o == me && e2 < tid);
        }
        a.order[rank] = tid;
    }
    __syncthreads();
    if (tid < 64) {                                    // exclusive scan of the totals
        int v[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[q] = tot[tid * 4 + q];
            sum += v[q];
        }
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (tid >= o) incl += y;
        }
        int ex = incl - sum;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid * 4 + q;
            if (e < a.E) {
                a.offsets[e] = ex;
                a.counts[e] = v[q];
            }
            tot[e] = ex;
            ex += v[q];
        }
        if (tid == 63) a.offsets[a.E] = incl;
    }
    __syncthreads();
    if (tid < 256) {                                   // range offsets: expert offset + earlier ranges
        int run = tot[tid];
        for (int w = 0; w < PW; ++w) {
            const int c = cw[w][tid];
            cw[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    int* off = cw[wave];
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int base = i0; base < i1; base += 64) {
        const int i = base + lane;
        const bool valid = i < i1;
        const int e = valid ? a.route[i] : 0x1FF;       // 9 bits: never a real expert
        uint64_t same = ~0ull;
#pragma unroll
        for (int b = 0; b < 9; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        if (valid) {
            const int slot = off[e] + __popcll(same & lt);
            a.perm_tok[slot] = i / a.k;
            a.slot_of[i] = slot;
            const uint64_t higher = lane == 63 ? 0ull : (same >> (lane + 1));
            if (higher == 0) off[e] += __popcll(same);
        }
    }
}

// h[t] += sum_j gate[t][j] * y[slot_of[t][j]]  (j in selection order)
__global__ __launch_bounds__(256) void combine_kernel(MoeArgs a) {
    const long t = blockIdx.x;
    float gt[16];
    long yo[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        gt[j] = j < a.k ? a.gates[t * a.k + j] : 0.f;
        yo[j] = j < a.k ? (long)a.slot_of[t * a.k + j] * a.d : 0;
    }
    float* hr = a.h + t * a.d;
    // blockIdx.y: a 1024-column slice of the row, one float4 per thread
    for (int c = (blockIdx.y * 256 + threadIdx.x) * 4; c < min(a.d, (int)(blockIdx.y + 1) * 1024);
         c += 1024) {
        float4 acc = *reinterpret_cast<const float4*>(hr + c);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j < a.k) {
                const float4 y = *reinterpret_cast<const float4*>(a.y + yo[j] + c);
                acc.x += gt[j] * y.x;
                acc.y += gt[j] * y.y;
                acc.z += gt[j] * y.z;
                acc.w += gt[j] * y.w;
            }
        }
        *reinterpret_cast<float4*>(hr + c) = acc;
    }
}

// The same with the number of experts per token known at compile time: the
// K expert rows' loads go out together, then the adds run in the same order
// as above.
template <int K>
__global__ __launch_bounds__(256) void combine_k_kernel(MoeArgs a) {
    const long t = blockIdx.x;
    float gt[K];
    long yo[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        gt[j] = a.gates[t * K + j];
        yo[j] = (long)a.slot_of[t * K + j] * a.d;
    }
    float* hr = a.h + t * a.d;
    for (int c = (blockIdx.y * 256 + threadIdx.x) * 4; c < min(a.d, (int)(blockIdx.y + 1) * 1024);
         c += 1024) {
        float4 y[K];
#pragma unroll
        for (int j = 0; j < K; ++j) y[j] = *reinterpret_cast<const float4*>(a.y + yo[j] + c);
        float4 acc = *reinterpret_cast<const float4*>(hr + c);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            acc.x += gt[j] * y[j].x;
            acc.y += gt[j] * y[j].y;
            acc.z += gt[j] * y[j].z;
            acc.w += gt[j] * y[j].w;
        }
        *reinterpret_cast<float4*>(hr + c) = acc;
    }
}

}  // namespace

hipError_t moe_route(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    hipLaunchKernelGGL(route_kernel, dim3(cdiv(a.T, 4)), dim3(256), 0, st, a);
    if ((long)a.T * a.k <= 8192) {
        // few assignments (a canvas): one workgroup places them all
        hipLaunchKernelGGL(place_all_kernel, dim3(1), dim3(64 * PW), 0, st, a);
    } else {
        hipLaunchKernelGGL(count_kernel, dim3(a.E), dim3(256), 0, st, a);
        hipLaunchKernelGGL(place_kernel, dim3(a.E), dim3(64), 0, st, a);
        if (a.order) hipLaunchKernelGGL(order_kernel, dim3(1), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

// the ring kernel needs whole rings of four 64-wide stages in both products
bool expert_dma_ok(const MoeArgs& a) {
    static int enabled = -1;
    if (enabled < 0) {
        const char* e = getenv("DG_DMA");
        enabled = e ? atoi(e) : 1;
    }
    // DG_DMA=0 (sweeps) turns off the bf16 ring only: 8-bit experts run on
    // the ring alone
    return (enabled || a.f8 || a.f4) && a.d % 256 == 0 && a.F % 256 == 0;
}

template <typename T>
hipError_t moe_gateup(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.f4) {
        if (sizeof(T) != 2 || !expert_dma_ok(a) || !a.x_gate || !a.x_up) return hipErrorInvalidValue;
        hipLaunchKernelGGL((expert_dma_kernel<0, 2>), dim3(cdiv(a.F, 128), a.E), dim3(256), 0, st, a);
    } else if (a.f8) {
        if (sizeof(T) != 2 || !expert_dma_ok(a)) return hipErrorInvalidValue;
        hipLaunchKernelGGL((expert_dma_kernel<0, 1>), dim3(cdiv(a.F, 64), a.E), dim3(256), 0, st, a);
    } else if (sizeof(T) == 2 && expert_dma_ok(a))
        hipLaunchKernelGGL((expert_dma_kernel<0, 0>), dim3(cdiv(a.F, 32), a.E), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((expert_kernel<T, 0>), dim3(cdiv(a.F, 32), a.E), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t moe_down(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.f4) {
        if (sizeof(T) != 2 || !expert_dma_ok(a) || !a.x_down) return hipErrorInvalidValue;
        hipLaunchKernelGGL((expert_dma_kernel<1, 2>), dim3(cdiv(a.d, 256), a.E), dim3(256), 0, st, a);
    } else if (a.f8) {
        if (sizeof(T) != 2 || !expert_dma_ok(a)) return hipErrorInvalidValue;
        hipLaunchKernelGGL((expert_dma_kernel<1, 1>), dim3(cdiv(a.d, 128), a.E), dim3(256), 0, st, a);
    } else if (sizeof(T) == 2 && expert_dma_ok(a))
        hipLaunchKernelGGL((expert_dma_kernel<1, 0>), dim3(cdiv(a.d, 64), a.E), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((expert_kernel<T, 1>), dim3(cdiv(a.d, 32), a.E), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t moe_combine(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    const dim3 grid(a.T, cdiv(a.d, 1024));
    if (a.k == 8)
        hipLaunchKernelGGL(combine_k_kernel<8>, grid, dim3(256), 0, st, a);
    else if (a.k == 4)
        hipLaunchKernelGGL(combine_k_kernel<4>, grid, dim3(256), 0, st, a);
    else if (a.k == 2)
        hipLaunchKernelGGL(combine_k_kernel<2>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template hipError_t moe_gateup<bf16_t>(const MoeArgs&, hipStream_t);
template hipError_t moe_gateup<float>(const MoeArgs&, hipStream_t);
template hipError_t moe_down<bf16_t>(const MoeArgs&, hipStream_t);
template hipError_t moe_down<float>(const MoeArgs&, hipStream_t);

}  // namespace dg
