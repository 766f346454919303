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

// Top-k of token t's E logits z (global or LDS) by one wave: k rounds of a
// wave-wide max over (logit, -index); gates = softmax over the selected
// logits in selection order.
__device__ __forceinline__ void route_select(const MoeArgs& a, long t, const float* z, int lane) {
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
    const float z0 = __shfl(myz, 0, 64);
    const float ex = lane < a.k ? expf(myz - z0) : 0.f;
    const float s = wave_sum(ex);
    if (lane < a.k) {
        a.route[t * a.k + lane] = mye;
        a.gates[t * a.k + lane] = ex / s;
    }
}

// One wave per token, logits z [T][E] from the router product.
__global__ __launch_bounds__(256) void route_kernel(MoeArgs a) {
    const int lane = threadIdx.x & 63;
    const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;
    route_select(a, t, a.z + t * a.E, lane);
}

// Router logits and top-k of one token per workgroup, for canvas-sized
// batches, where a split-K router product, its epilogue and route_kernel
// are three launches of a few microseconds each.  z[e] = sum_k u[k] W[e][k]
// in fp32 (u the fp32 normalised token, W the bf16 router rows widened on
// load): lane l owns the 8-wide pieces k = 512 c + 8 l (c < NCH = d / 512)
// and keeps the token's pieces in registers.  Wave w of 8 takes the groups
// of 4 experts w, w + 8, ... (in a rotated order), each group's weights loaded
// while the previous group is multiplied; a fixed butterfly sums each
// expert's 64 lane partials, so the order of the groups changes no bit.  Every workgroup reads all E x d router weights, which stay in
// L2.
template <int NCH>
struct RouterGroup {
    uint4 w[4][NCH];
};

template <int NCH>
__device__ __forceinline__ void router_load(RouterGroup<NCH>& g, const uint16_t* wr, int grp, int E,
                                            int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = min(4 * grp + i, E - 1);   // rows past E repeat the last (unused)
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            g.w[i][c] = *reinterpret_cast<const uint4*>(wr + (long)e * (NCH * 512) + 512 * c + 8 * lane);
    }
}

// the group's four logits: lane l's partials, then lanes l ^ 32 and l ^ 16
// swap halves so that lane l keeps expert 2 (l / 32) + (l / 16) mod 2, then
// sums over l ^ 8, ^ 4, ^ 2, ^ 1; lanes 0, 16, 32, 48 write experts 0..3
template <int NCH>
__device__ __forceinline__ void router_group(const RouterGroup<NCH>& g, const float (&u)[NCH][8],
                                             int grp, int E, int lane, float* zs) {
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint32_t q[4] = {g.w[i][c].x, g.w[i][c].y, g.w[i][c].z, g.w[i][c].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc = __builtin_fmaf(u[c][2 * j], __uint_as_float(q[j] << 16), acc);
                acc = __builtin_fmaf(u[c][2 * j + 1], __uint_as_float(q[j] & 0xFFFF0000u), acc);
            }
        }
        p[i] = acc;
    }
    const bool hi32 = lane & 32, hi16 = lane & 16;
    // lanes below 32 keep experts 0, 1 and send 2, 3; the others the reverse
    const float s0 = hi32 ? p[0] : p[2], s1 = hi32 ? p[1] : p[3];
    const float r0 = __shfl_xor(s0, 32, 64), r1 = __shfl_xor(s1, 32, 64);
    const float k0 = (hi32 ? p[2] : p[0]) + r0, k1 = (hi32 ? p[3] : p[1]) + r1;
    const float s = hi16 ? k0 : k1;
    const float r = __shfl_xor(s, 16, 64);
    float v = (hi16 ? k1 : k0) + r;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) v = v + __shfl_xor(v, o, 64);
    const int e = 4 * grp + 2 * (hi32 ? 1 : 0) + (hi16 ? 1 : 0);
    if ((lane & 15) == 0 && e < E) zs[e] = v;
}

constexpr int kRouterWaves = 8;

template <int NCH>
__global__ __launch_bounds__(64 * kRouterWaves) void router_route_kernel(MoeArgs a) {
    __shared__ float zs[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long t = blockIdx.x;
    const float* ur = a.router_u + t * (NCH * 512);
    const uint16_t* wr = static_cast<const uint16_t*>(a.router_w);
    float u[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const float4 x0 = *reinterpret_cast<const float4*>(ur + 512 * c + 8 * lane);
        const float4 x1 = *reinterpret_cast<const float4*>(ur + 512 * c + 8 * lane + 4);
        u[c][0] = x0.x;
        u[c][1] = x0.y;
        u[c][2] = x0.z;
        u[c][3] = x0.w;
        u[c][4] = x1.x;
        u[c][5] = x1.y;
        u[c][6] = x1.z;
        u[c][7] = x1.w;
    }
    // wave w owns groups w + W j (j < nj, W waves); workgroup t starts at
    // j = t mod nj, so that the workgroups of an XCD, which run side by side,
    // read different weight rows at a time rather than the same lines in
    // lockstep
    constexpr int W = kRouterWaves;
    const int ngroups = cdiv(a.E, 4);
    const int nj = wave < ngroups ? cdiv(ngroups - wave, W) : 0;
    const int rot = nj ? (int)(t % nj) : 0;
    auto grp = [&](int jj) { return wave + W * ((jj + rot) % nj); };
    RouterGroup<NCH> ga, gb;
    int jj = 0;
    if (jj < nj) router_load(ga, wr, grp(jj), a.E, lane);
    // two groups a trip: the next group's loads go out before this one's
    // products
    while (jj < nj) {
        if (jj + 1 < nj) router_load(gb, wr, grp(jj + 1), a.E, lane);
        router_group(ga, u, grp(jj), a.E, lane, zs);
        ++jj;
        if (jj >= nj) break;
        if (jj + 1 < nj) router_load(ga, wr, grp(jj + 1), a.E, lane);
        router_group(gb, u, grp(jj), a.E, lane, zs);
        ++jj;
    }
    __syncthreads();
    if (wave == 0) route_select(a, t, zs, lane);
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

// work[r] for r = 0 .. E: exclusive prefix of ch[0 .. E) (chunks of the
// expert of rank r, in LDS), by threads 0..63 of the block, four each; also
// into the LDS array lw[0 .. E) when it is given.
__device__ __forceinline__ void write_work(const int* ch, int E, int32_t* work, int* lw = nullptr) {
    const int tid = threadIdx.x;
    if (tid >= 64) return;
    int v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[q] = tid * 4 + q < E ? ch[tid * 4 + q] : 0;
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
        if (tid * 4 + q < E) {
            work[tid * 4 + q] = ex;
            if (lw) lw[tid * 4 + q] = ex;
        }
        ex += v[q];
    }
    if (tid == 63) work[E] = incl;
}

// The records of rank r's work items: expert e, its first routed row off
// and row count cnt, its first item `first`; one record per chunk.
__device__ __forceinline__ void write_rank_items(const MoeArgs& a, int e, int off, int cnt, int first) {
    for (int i = 0; i * kMoeChunk < cnt; ++i)
        reinterpret_cast<int4*>(a.items)[first + i] = make_int4(e, off, i * kMoeChunk, cnt);
}

// The work items' records (a.items), from order, offsets and work once an
// earlier kernel, or this workgroup before a barrier, has written them: the
// threads take the ranks in turn.
__device__ __forceinline__ void write_items(const MoeArgs& a) {
    for (int r = threadIdx.x; r < a.E; r += blockDim.x) {
        const int e = a.order[r];
        const int off = a.offsets[e];
        write_rank_items(a, e, off, a.offsets[e + 1] - off, a.work[r]);
    }
}

// The rank of work item w's expert when no records were written: a binary
// search of work[] (work[r] <= w < work[r + 1]).
__device__ __forceinline__ int item_rank(const MoeArgs& a, int w) {
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.work[mid] <= w)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Experts by falling count (ties: lower id) from the counts, and the chunk
// prefix over that order.
__global__ __launch_bounds__(256) void order_kernel(MoeArgs a) {
    __shared__ int ch[256];
    const int e = threadIdx.x;
    if (e < a.E) {
        const int me = a.counts[e];
        int rank = 0;
        for (int e2 = 0; e2 < a.E; ++e2) {
            const int o = a.counts[e2];
            rank += (o > me) || (o == me && e2 < e);
        }
        a.order[rank] = e;
        ch[rank] = cdiv(me, kMoeChunk);
    }
    if (!a.work) return;
    __syncthreads();
    write_work(ch, a.E, a.work);
    if (!a.items) return;
    __syncthreads();
    write_items(a);
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
// weights: 64 rows (two halves of 32 columns) per block.  (Quantised
// experts run on the block-scaled MFMA kernels of moe_mx.hip.)
struct XdCtx {
    int e, off, cnt, K, NOUT, c0, n, rot;
    int m0, m1;              // the token range [m0, m1) of the expert this block runs
    int lane, wave, r16, g4, ct, mp, lr, lc;
    const char* wsrc[2];     // byte addresses of this lane's weight chunks at k = 0
    const bf16_t* X;
};

template <int MODE, int G>
__device__ __forceinline__ void expert_groups(const MoeArgs& a, const XdCtx& c, unsigned char* w0,
                                              unsigned char* w1, unsigned char* w2, unsigned char* w3,
                                              unsigned char* x0, unsigned char* x1, unsigned char* x2,
                                              unsigned char* x3) {
    constexpr int WQ = 2;                              // weight DMAs per wave per stage
    constexpr int PER = WQ + G;                        // DMAs per wave per stage
    constexpr int WSTAGE = 128;                        // weight bytes per row and stage
    constexpr int J = 1;                               // 16-column tiles per half and wave
    constexpr int HALF = 32 * J;                       // columns per half of the block
    const int n = c.n, rot = c.rot, mp = c.mp, ct = c.ct, r16 = c.r16, g4 = c.g4;
    const int wblk = c.wave * WQ * 1024;
    const int xblk = c.wave * G * 1024;
    const int roff = r16 * 128;
    // output columns of the lane (tile ct + 2j of the first half; the
    // second half is the up projection, or the down columns HALF later)
    int col[J];
#pragma unroll
    for (int j = 0; j < J; ++j) col[j] = c.c0 + (ct + 2 * j) * 16 + r16;
    for (int mg = c.m0; mg < c.m1; mg += 32 * G) {
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

#define XD_ISSUE(ST, WB, XB)                                                                      \
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
        }
        // fragments: token rows 16*(mp + 2q) + r16; weight rows (ct + 2j)*16
        // + r16 of each half; k-step s of a lane is chunk 4*s + g4 of both
        // operands
#define XD_COMPUTE(WB, XB)                                                                        \
        {                                                                                         \
            u32x4 fga[J], fgb[J], fua[J], fub[J], fxa[G], fxb[G];                                 \
            const uint32_t xa = lds_addr(XB) + (16 * mp) * 128 + roff;                            \
            const int xs = r16 & 7;                                                               \
            const uint32_t sa = (g4 ^ xs) << 4;                                                   \
            const uint32_t sb = ((4 + g4) ^ xs) << 4;                                             \
            {                                                                                     \
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
#define XD_STAGE(t, CW, CX, NW, NX)                          \
        {                                                    \
            if ((t) + 2 < n)                                 \
                DG_WAIT_VM(2 * PER);                         \
            else if ((t) + 1 < n)                            \
                DG_WAIT_VM(PER);                             \
            else                                             \
                DG_WAIT_VM(0);                               \
            barrier_lds();                                   \
            if ((t) + 3 < n) XD_ISSUE((t) + 3, NW, NX);      \
            XD_COMPUTE(CW, CX);                              \
        }
        XD_ISSUE(0, w0, x0);
        XD_ISSUE(1, w1, x1);
        XD_ISSUE(2, w2, x2);
        for (int t = 0; t < n; t += 4) {
            XD_STAGE(t, w0, x0, w3, x3);
            XD_STAGE(t + 1, w1, x1, w0, x0);
            XD_STAGE(t + 2, w2, x2, w1, x1);
            XD_STAGE(t + 3, w3, x3, w2, x2);
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
                        const float gv = ag[q][j][i];
                        const float uv = au[q][j][i];
                        const float sv = gv / (1.0f + __expf(-gv));
                        reinterpret_cast<bf16_t*>(a.act)[(long)(c.off + row) * a.F + col[j]] =
                            f2bf(sv * uv);
                    } else {
                        a.y[(long)(c.off + row) * a.d + col[j]] = ag[q][j][i];
                        if (col[j] + HALF < c.NOUT)
                            a.y[(long)(c.off + row) * a.d + col[j] + HALF] = au[q][j][i];
                    }
                }
            }
        }
        // the next group's loads refill the ring only after every wave is done
        barrier_lds();
    }
}

// Blocks of 64 weight rows (gate and up rows of 32 columns (MODE 0) or 64
// columns of the down projection (MODE 1)).  With the routing's work items
// (`work`), blockIdx.y is one item: a chunk of up to 64 tokens of one expert,
// the busiest experts' chunks first, so the chunks of a busy expert run side
// by side instead of one block walking them in turn (under collapsed
// routing one expert takes hundreds of tokens).  Without them, blockIdx.y is
// an expert (in `order` when set) and the block walks all its tokens.  A
// chunk of at most 32 tokens runs one 32-token group, a larger one one group
// of 64.
template <int MODE>
__global__ __launch_bounds__(256) void expert_dma_kernel(MoeArgs a) {
    if (a.halt && *a.halt) return;
    __shared__ __align__(1024) unsigned char w0[64 * 128], x0[8192];
    __shared__ __align__(1024) unsigned char w1[64 * 128], x1[8192];
    __shared__ __align__(1024) unsigned char w2[64 * 128], x2[8192];
    __shared__ __align__(1024) unsigned char w3[64 * 128], x3[8192];
    constexpr int HALF = 32;                           // columns per half of a block

    XdCtx c;
    if (a.work && a.order) {
        const int w = blockIdx.y;
        if (w >= a.work[a.E]) return;
        if (a.items) {
            const int4 it = reinterpret_cast<const int4*>(a.items)[w];
            c.e = it.x;
            c.off = it.y;
            c.m0 = it.z;
            c.cnt = it.w;
        } else {
            const int lo = item_rank(a, w);
            c.e = a.order[lo];
            c.off = a.offsets[c.e];
            c.cnt = a.offsets[c.e + 1] - c.off;
            c.m0 = (w - a.work[lo]) * kMoeChunk;
        }
        c.m1 = min(c.cnt, c.m0 + kMoeChunk);
    } else {
        // the busiest experts first, so their longer blocks do not form the tail
        c.e = a.order ? a.order[blockIdx.y] : (int)blockIdx.y;
        c.off = a.offsets[c.e];
        c.cnt = a.offsets[c.e + 1] - c.off;
        c.m0 = 0;
        c.m1 = c.cnt;
    }
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
        {
            const int r = (c.wave * 2 + q) * 8 + c.lr;             // row within the block
            const int rr = MODE == 0 ? (r & (HALF - 1)) : r;
            const int col = min(c.c0 + rr, c.NOUT - 1);
            const char* base = (MODE == 0 && r >= HALF) ? Wu : Wg;
            c.wsrc[q] = base + (((long)c.e * c.NOUT + col) * c.K + c.lc) * 2;
        }
    }
    if (__builtin_amdgcn_readfirstlane(c.m1 - c.m0) <= 32)
        expert_groups<MODE, 1>(a, c, w0, w1, w2, w3, x0, x1, x2, x3);
    else
        expert_groups<MODE, 2>(a, c, w0, w1, w2, w3, x0, x1, x2, x3);
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
    __shared__ int ch[256];        // chunks of the expert of each rank
    __shared__ int ord[256];       // the expert of each rank
    __shared__ int wk[256];        // the first work item of each rank
    __shared__ int cnt[256];       // per-expert totals, kept through the scan
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
        ord[rank] = tid;
        ch[rank] = cdiv(me, kMoeChunk);
    }
    __syncthreads();
    if (a.order && a.work) write_work(ch, a.E, a.work, wk);
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
            cnt[e] = v[q];
            ex += v[q];
        }
        if (tid == 63) a.offsets[a.E] = incl;
    }
    __syncthreads();
    if (a.order && a.work && a.items)                  // the records, from LDS
        for (int r = tid; r < a.E; r += 64 * PW) {
            const int e = ord[r];
            write_rank_items(a, e, tot[e], cnt[e], wk[r]);
        }
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

// The combine, with the next layer's attention RMSNorm of the new rows
// fused: one workgroup a token takes the whole row (thread t the float4 at
// 4t + 1024 i, the layout of rmsnorm_kernel), adds the K expert rows in the
// order combine_k_kernel adds them, writes h and normalises it with the
// shared RMSNorm arithmetic, so both h and u have the bits of the two
// separate kernels.
template <int K, typename T>
__global__ __launch_bounds__(256) void combine_norm_k_kernel(MoeArgs a, const float* __restrict__ nw,
                                                             T* __restrict__ u, float eps) {
    const long t = blockIdx.x;
    float gt[K];
    long yo[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        gt[j] = a.gates[t * K + j];
        yo[j] = (long)a.slot_of[t * K + j] * a.d;
    }
    float* hr = a.h + t * a.d;
    float ss = 0.f;
    for (int c = threadIdx.x * 4; c < a.d; c += 1024) {
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
        ss = rms_accum(ss, acc);
    }
    __shared__ float part[4];
    const float scale = rms_block_scale(ss, part, a.d, eps);
    T* o = u + t * a.d;
    for (int c = threadIdx.x * 4; c < a.d; c += 1024) {
        const float4 r = rms_apply(*reinterpret_cast<const float4*>(hr + c), scale, nw, c);
        o[c + 0] = Elt<T>::from_f(r.x);
        o[c + 1] = Elt<T>::from_f(r.y);
        o[c + 2] = Elt<T>::from_f(r.z);
        o[c + 3] = Elt<T>::from_f(r.w);
    }
}

}  // namespace

bool moe_combine_norm_ok(int k) { return k == 2 || k == 4 || k == 8; }

template <typename T>
hipError_t moe_combine_norm(const MoeArgs& a, const float* nw, T* u, float eps, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.d % 4) return hipErrorInvalidValue;
    const dim3 grid(a.T);
    if (a.k == 8)
        hipLaunchKernelGGL((combine_norm_k_kernel<8, T>), grid, dim3(256), 0, st, a, nw, u, eps);
    else if (a.k == 4)
        hipLaunchKernelGGL((combine_norm_k_kernel<4, T>), grid, dim3(256), 0, st, a, nw, u, eps);
    else if (a.k == 2)
        hipLaunchKernelGGL((combine_norm_k_kernel<2, T>), grid, dim3(256), 0, st, a, nw, u, eps);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}
template hipError_t moe_combine_norm<bf16_t>(const MoeArgs&, const float*, bf16_t*, float, hipStream_t);
template hipError_t moe_combine_norm<float>(const MoeArgs&, const float*, float*, float, hipStream_t);

hipError_t moe_route(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.router_w) {
        if (!a.router_u || !router_fused_ok(a.T, a.d, a.E)) return hipErrorInvalidValue;
        switch (a.d / 512) {
            case 1: hipLaunchKernelGGL(router_route_kernel<1>, dim3(a.T), dim3(64 * kRouterWaves), 0, st, a); break;
            case 2: hipLaunchKernelGGL(router_route_kernel<2>, dim3(a.T), dim3(64 * kRouterWaves), 0, st, a); break;
            case 4: hipLaunchKernelGGL(router_route_kernel<4>, dim3(a.T), dim3(64 * kRouterWaves), 0, st, a); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        hipLaunchKernelGGL(route_kernel, dim3(cdiv(a.T, 4)), dim3(256), 0, st, a);
    }
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
    return a.d % 256 == 0 && a.F % 256 == 0;
}

// blockIdx.y of the ring kernels: the most work items there can be (every
// expert's last chunk partial), or the experts
static int dma_rows(const MoeArgs& a) {
    return a.work && a.order ? cdiv(a.T * a.k, kMoeChunk) + std::min(a.E, a.T * a.k) : a.E;
}

template <typename T>
hipError_t moe_gateup(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.f4 || a.f8) {
        if (sizeof(T) != 2) return hipErrorInvalidValue;
        return moe_gateup_mx(a, st);
    }
    if (sizeof(T) == 2 && expert_dma_ok(a))
        hipLaunchKernelGGL((expert_dma_kernel<0>), dim3(cdiv(a.F, 32), dma_rows(a)), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((expert_kernel<T, 0>), dim3(cdiv(a.F, 32), a.E), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t moe_down(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.f4 || a.f8) {
        if (sizeof(T) != 2) return hipErrorInvalidValue;
        return moe_down_mx(a, st);
    }
    if (sizeof(T) == 2 && expert_dma_ok(a))
        hipLaunchKernelGGL((expert_dma_kernel<1>), dim3(cdiv(a.d, 64), dma_rows(a)), dim3(256), 0, st, a);
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
