// C ABI of the denoising step (include/dg.h): argument checks, workspace
// layout, and the order of kernel launches for encode, denoise, sample,
// commit and the block loop.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dg.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

dg_status fail(dg_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

#define DG_HIP(expr)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (expr);                                                          \
        if (e_ != hipSuccess)                                                            \
            return fail(DG_ERR_HIP, "%s: %s (%s:%d)", #expr, hipGetErrorString(e_),      \
                        __FILE__, __LINE__);                                             \
    } while (0)

#define DG_TRY(expr)                     \
    do {                                 \
        dg_status s_ = (expr);           \
        if (s_ != DG_OK) return s_;      \
    } while (0)

// ---- kernel timers (dg_timer_enable / dg_timer_read)
struct Timers {
    uint32_t mask = 0;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[DG_TIMER_COUNT];
    void clear() {
        for (auto& v : ev) {
            for (auto& p : v) {
                (void)hipEventDestroy(p.first);
                (void)hipEventDestroy(p.second);
            }
            v.clear();
        }
    }
};
Timers g_timers;

// Runs `launch` (returning hipError_t) between two events on `st` if timer
// `id` is enabled.
template <typename F>
hipError_t timed(int id, hipStream_t st, F&& launch) {
    if (!(g_timers.mask & (1u << id))) return launch();
    hipEvent_t a, b;
    hipError_t e = hipEventCreate(&a);
    if (e != hipSuccess) return e;
    e = hipEventCreate(&b);
    if (e != hipSuccess) return e;
    e = hipEventRecord(a, st);
    if (e != hipSuccess) return e;
    e = launch();
    if (e != hipSuccess) return e;
    e = hipEventRecord(b, st);
    g_timers.ev[id].push_back({a, b});
    return e;
}

constexpr int kEncodeTokens = 4096;    // tokens per encode chunk (all sequences)
constexpr int kAttnPartRows = 8192;    // split-KV partial rows budget
constexpr int kMaxSplitsSC = 64;       // self-conditioning split-K limit

size_t elt_size(int dtype) { return dtype == DG_BF16 ? 2 : 4; }

// Bump allocator over the caller's workspace (256-byte aligned pieces).
struct Carver {
    char* base;
    size_t size, off = 0;
    bool ok = true;
    Carver(void* b, size_t s) : base((char*)b), size(s) {}
    template <typename T>
    T* take(size_t n) {
        off = (off + 255) & ~(size_t)255;
        size_t bytes = n * sizeof(T);
        T* p = base ? (T*)(base + off) : nullptr;
        off += bytes;
        if (base && off > size) ok = false;
        return p;
    }
    void* take_bytes(size_t n) { return take<char>(n); }
};

}  // namespace

struct dg_model {
    dg_config c;
    const void* embed;
    const void* embed_t;
    const void* embed_head;   // optional: E in the blocked layout (dg_embed_head)
    // bf16, d % 256 == 0, V % 128 == 0: the vocabulary products run on the
    // ring kernel with both operands in the blocked layout (embed_t is E^T
    // blocked; the activations are written blocked)
    bool blocked = false;
    const void* w_sc;
    const float* final_norm;
    std::vector<dg_layer_weights> layers;
    // block loop: pinned host memory that the sampler's canvas kernel writes
    // the stop flags of two rounds into, and the events that say they have
    // arrived (created with the model)
    int32_t* hflags = nullptr;
    int hflags_cap = 0;
    hipEvent_t flag_ev[2] = {nullptr, nullptr};
    ~dg_model() {
        if (hflags) (void)hipHostFree(hflags);
        for (hipEvent_t e : flag_ev)
            if (e) (void)hipEventDestroy(e);
    }
};

struct dg_kv {
    int B, cap, len;
    void* buf;
};

namespace {

// Per-call scratch, carved in a fixed order so a size query and a real call
// agree.
struct Scratch {
    float* h;
    void* u;
    float* qkv;
    void* q;
    void* ao;
    float* part_o;
    float* part_ml;
    float* z;
    int32_t* route;
    float* gates;
    int32_t* counts;
    int32_t* offsets;
    int32_t* order;
    int32_t* perm_tok;
    int32_t* slot_of;
    void* act;
    float* y;
    float* sc_part;
    void* sc_s;
    int32_t* tok;
    float* gp;        // split-K partials of the small projections
    void* probs;      // bf16 models: softmax(prev logits) in bf16 for self-conditioning
    void* ut;         // blocked models: final-normed rows for the head, blocked layout
    int ut_rows = 0;  // rows `ut` holds (the canvas tokens, padded to 256)
    int probs_tiled = 0;  // `probs` in the 64-wide blocked layout (else row-major)
    float* u32;       // bf16 models: fp32 normalised activations for the router
    // quantised experts: MXFP8 codes and scale codes of the normalised tokens
    // and of the gate/up output
    uint8_t* u8 = nullptr;
    uint8_t* u8s = nullptr;
    uint8_t* act8 = nullptr;
    uint8_t* act8s = nullptr;
    int32_t* work = nullptr;  // expert chunk prefix over the busiest-first order
    int32_t* items = nullptr;      // the work items' records (4 words each)
    float* tmax;      // blocked models: head GEMM row maxima per 64-column slab
    // set by the block loop (not carved): the head GEMM writes its slab
    // maxima (fuse), and the probabilities of the previous round's logits are
    // already in `probs`, written by the sampler (probs_ready)
    bool fuse = false;
    bool probs_ready = false;
    // top-k self-conditioning: the previous round's candidates and weights
    // (written by the sampler in the block loop: topk_ready), and whether
    // the head writes its slab maxima for the sampler
    int topk = 0;
    bool topk_ready = false;
    bool want_rowmax = false;
    int32_t* tk_idx;  // [canvas tokens][kTopKMax]
    float* tk_p;
    int32_t* zero;    // one int32 kept at 0 (the stop flag of a list-only pass)
    // set by the block loop (not carved): when *halt != 0 every sequence of
    // the batch has stopped and the heavy kernels of a round skip their work
    const int32_t* halt = nullptr;
};

int token_budget(const dg_model* m, int B) {
    return std::max(B * m->c.canvas, std::max(kEncodeTokens, B));
}

int sc_splits(const dg_model* m, int T) {
    // enough workgroups for the chip on the [T x d] output tiles; a multiple
    // of 8 so the column tiles of one split can share an XCD
    const int tiles = cdiv(T, 256) * cdiv(m->c.d_model, 256);
    int s = std::max(1, std::min(kMaxSplitsSC, 256 / std::max(tiles, 1)));
    return s >= 8 ? (s / 8) * 8 : s;
}

// Split-K partial budget of the small projections (floats): splits are chosen
// so that splits * tiles stays below ~640 workgroups of 64 columns x 256 rows.
constexpr size_t kSplitPartFloats = (size_t)640 * 64 * 256;

bool carve_scratch(Carver& cv, const dg_model* m, int B, Scratch& s) {
    const dg_config& c = m->c;
    const size_t es = elt_size(c.dtype);
    const size_t T = (size_t)token_budget(m, B);
    const size_t Tc = (size_t)B * c.canvas;
    const size_t qkvw = (size_t)(c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
    s.h = cv.take<float>(T * c.d_model);
    s.u = cv.take_bytes(T * c.d_model * es);
    s.qkv = cv.take<float>(T * qkvw);
    s.q = cv.take_bytes(T * c.n_heads * c.head_dim * es);
    s.ao = cv.take_bytes(T * c.n_heads * c.head_dim * es);
    // split-KV partials: up to eight splits of every canvas row
    const size_t prow = std::max<size_t>(kAttnPartRows, 8 * Tc);
    s.part_o = cv.take<float>(prow * c.n_heads * c.head_dim);
    s.part_ml = cv.take<float>(prow * c.n_heads * 2);
    s.z = cv.take<float>(T * c.n_experts);
    s.route = cv.take<int32_t>(T * c.top_k);
    s.gates = cv.take<float>(T * c.top_k);
    s.counts = cv.take<int32_t>(c.n_experts);
    s.order = cv.take<int32_t>(c.n_experts);
    s.offsets = cv.take<int32_t>(c.n_experts + 1);
    // (16 entries of padding: the block-scaled expert kernels read a wave's
    // 16 sorted slots with scalar loads, up to 15 past an expert's last slot)
    s.perm_tok = cv.take<int32_t>(T * c.top_k + 16);
    s.slot_of = cv.take<int32_t>(T * c.top_k);
    s.act = cv.take_bytes(T * c.top_k * c.d_ff * es);
    s.y = cv.take<float>(T * c.top_k * c.d_model);
    s.sc_part = cv.take<float>((size_t)sc_splits(m, (int)Tc) * Tc * c.d_model);
    s.sc_s = cv.take_bytes(Tc * c.d_model * es);
    s.gp = cv.take<float>(kSplitPartFloats);
    // rows padded to 256 for the blocked layout
    const size_t Tp = (size_t)cdiv((int)Tc, 256) * 256;
    s.probs = c.dtype == DG_BF16 ? cv.take_bytes(Tp * c.vocab * 2) : nullptr;
    s.probs_tiled = m->blocked ? 1 : 0;
    s.ut = m->blocked ? cv.take_bytes(Tp * c.d_model * 2) : nullptr;
    s.ut_rows = m->blocked ? (int)Tp : 0;
    s.tok = cv.take<int32_t>(T);
    const bool wide = c.dtype == DG_BF16;
    s.u32 = wide ? cv.take<float>(T * c.d_model) : nullptr;
    if (c.expert_dtype == DG_FP8_E4M3 || c.expert_dtype == DG_MXFP4) {
        s.u8 = cv.take<uint8_t>(T * c.d_model);
        s.u8s = cv.take<uint8_t>(T * c.d_model / 32);
        s.act8 = cv.take<uint8_t>(T * c.top_k * c.d_ff);
        s.act8s = cv.take<uint8_t>(T * c.top_k * c.d_ff / 32);
    }
    // the expert kernels' work items (chunks of up to 64 tokens of an expert)
    // and their records
    s.work = cv.take<int32_t>(c.n_experts + 1);
    s.items = cv.take<int32_t>(4 * ((T * c.top_k + dg::kMoeChunk - 1) / dg::kMoeChunk + c.n_experts));
    s.tmax = m->blocked ? cv.take<float>(Tc * (size_t)(c.vocab / 64)) : nullptr;
    s.tk_idx = cv.take<int32_t>(Tc * dg::kTopKMax);
    s.tk_p = cv.take<float>(Tc * dg::kTopKMax);
    s.zero = cv.take<int32_t>(64);
    return cv.ok;
}

dg_status check_ws(const dg_model* m, int B, void* ws, size_t bytes, Scratch& s, Carver& cv) {
    if (!ws) return fail(DG_ERR_ARG, "workspace is NULL");
    if (!carve_scratch(cv, m, B, s))
        return fail(DG_ERR_CAPACITY, "workspace of %zu bytes is too small (need %zu)", bytes,
                    cv.off);
    return DG_OK;
}

// layer pointers into the KV buffer
void kv_layer(const dg_model* m, const dg_kv* kv, int layer, void** kc, void** vc) {
    const dg_config& c = m->c;
    const size_t es = elt_size(c.dtype);
    const size_t per_layer = (size_t)kv->B * c.n_kv_heads * kv->cap * c.head_dim;
    char* K = (char*)kv->buf;
    char* V = K + per_layer * c.n_layers * es;
    *kc = K + per_layer * layer * es;
    *vc = V + per_layer * layer * es;
}

template <typename T>
dg_status gemm(const dg::GemmArgs& g, int amode, int epi, int splits, hipStream_t st) {
    DG_HIP(dg::gemm_tn<T>(g, amode, epi, splits, st));
    return DG_OK;
}

// Optional epilogue of the stacked Q/K/V product: RoPE and the KV-cache write
// straight from the split-K partials, taken when the product runs split over
// K on the skinny kernel (`done` tells the caller; otherwise C holds q|k|v).
struct RopeEpi {
    void *q, *kc, *vc;
    int B, n, pos0, cap, Hq, Hkv, dh, rope_on;
    float theta;
    bool done;
};

// Optional epilogue of the O projection: the residual add and the MoE half's
// RMSNorm of the new rows in one pass over the split-K partials (same
// outputs as rmsnorm), taken like RopeEpi.
struct AddNormEpi {
    const float* w;
    void* u;
    float* u32;
    uint8_t *q8, *q8s;
    float eps;
    bool done;
};

// C (epi)= x W^T for x [M][K] (model dtype, or fp32 when T = float) and
// W [N][K]: C fp32 [M][ldc].  bf16 uses the streaming GEMM, fp32 the LDS-tiled
// one.  When the output has too few tiles to fill the chip, K is split and a
// second pass sums the partials in a fixed order (deterministic).
template <typename T>
dg_status linear(const void* x, int M, int K, const void* W, int N, float* C, long ldc, int epi,
                 Scratch& s, hipStream_t st, const void* E = nullptr,
                 const int32_t* tokens = nullptr, int vocab = 0, int b_bf16 = 0,
                 const void* B2 = nullptr, int n_b2 = 0, const void* B3 = nullptr, int n_b3 = 0,
                 RopeEpi* rope = nullptr, AddNormEpi* addnorm = nullptr) {
    dg::GemmArgs g;
    g.M = M;
    g.N = N;
    g.K = K;
    g.A = x;
    g.lda = K;
    g.B = W;
    g.ldb = K;
    g.C = C;
    g.ldc = ldc;
    g.k_split = K;
    g.E = E;
    g.lde = N;
    g.tokens = tokens;
    g.vocab = vocab;
    g.E_is_f32 = sizeof(T) == 4;
    g.b_bf16 = b_bf16;
    g.B2 = B2;
    g.n_b2 = n_b2;
    g.B3 = B3;
    g.n_b3 = n_b3;
    const bool bf = sizeof(T) == 2;
    const int mt = bf ? cdiv(M, 16 * dg::stream_tm_for(M)) : cdiv(M, 64);
    long tiles_wide = (long)cdiv(N, 256) * mt;
    if (bf && tiles_wide >= 200) {
        DG_HIP(dg::gemm_stream(g, epi, 4, 1, st));
        return DG_OK;
    }
    if (bf) {
        // canvas-size bf16 projection: skinny ring kernel over 256 x 64 tiles,
        // split over K into 128-multiples, then the ordered split-K pass
        constexpr int target = 192;   // workgroups to aim for
        dg::GemmArgs p = g;
        const long stiles = (long)cdiv(N, 64) * cdiv(M, 256);
        int sp = (int)std::min<long>(std::max<long>(1, cdiv(target, (int)stiles)),
                                     std::max(1, K / 128));
        p.k_split = cdiv(cdiv(K, sp), 128) * 128;
        int used = cdiv(K, p.k_split);
        while (used > 1 && (size_t)used * M * N > kSplitPartFloats) {
            p.k_split += 128;
            used = cdiv(K, p.k_split);
        }
        p.C = s.gp;
        p.ldc = N;
        if ((size_t)used * M * N <= kSplitPartFloats && dg::gemm_skinny_ok(p)) {
            DG_HIP(dg::gemm_skinny_splitk(p, used, st));
            if (rope) {
                DG_HIP(dg::splitk_rope_kv<T>(s.gp, used, (T*)rope->q, (T*)rope->kc, (T*)rope->vc,
                                             rope->B, rope->n, rope->pos0, rope->cap, rope->Hq,
                                             rope->Hkv, rope->dh, rope->rope_on, rope->theta, st));
                rope->done = true;
            } else if (addnorm && epi == dg::EPI_ADD_F32 && ldc == N) {
                DG_HIP(dg::splitk_add_norm<T>(s.gp, used, C, M, N, addnorm->w, (T*)addnorm->u,
                                              addnorm->eps, st, addnorm->u32, addnorm->q8,
                                              addnorm->q8s));
                addnorm->done = true;
            } else {
                DG_HIP(dg::splitk_epilogue(g, s.gp, used, epi, st));
            }
            return DG_OK;
        }
    }
    const long tiles = (long)cdiv(N, 64) * mt;
    int splits = (int)std::min<long>(std::max<long>(1, cdiv(320, (int)tiles)), std::max(1, K / 64));
    while (splits > 1 && (size_t)splits * M * N > kSplitPartFloats) --splits;
    if (splits <= 1) {
        if (bf) DG_HIP(dg::gemm_stream(g, epi, 1, 1, st));
        else DG_HIP(dg::gemm_tn<T>(g, 0, epi, 1, st));
        return DG_OK;
    }
    dg::GemmArgs p = g;
    p.C = s.gp;
    p.ldc = N;
    p.k_split = cdiv(cdiv(K, splits), 64) * 64;
    const int used = cdiv(K, p.k_split);
    if (bf) DG_HIP(dg::gemm_stream(p, dg::EPI_SPLITK, 1, used, st));
    else DG_HIP(dg::gemm_tn<T>(p, 0, dg::EPI_SPLITK, used, st));
    DG_HIP(dg::splitk_epilogue(g, s.gp, used, epi, st));
    return DG_OK;
}

// attention RMSNorm weight of the layer after l (nullptr after the last)
static const float* next_attn_norm(const dg_model* m, int l) {
    return l + 1 < m->c.n_layers ? m->layers[l + 1].attn_norm : nullptr;
}

// ---- attention half-block: n new tokens per sequence at [pos0, pos0+n)
template <typename T>
dg_status attn_half(dg_model* m, dg_kv* kv, int layer, int B, int n, int pos0, int causal,
                    float* h, Scratch& s, hipStream_t st, bool normed = false,
                    AddNormEpi* moe_norm = nullptr) {
    const dg_config& c = m->c;
    const dg_layer_weights& L = m->layers[layer];
    const int Tn = B * n;
    const int d = c.d_model, dh = c.head_dim;
    const int qkvw = (c.n_heads + 2 * c.n_kv_heads) * dh;
    // (normed: the previous MoE half's combine has already written s.u)
    if (!normed) DG_HIP(dg::rmsnorm<T>(h, L.attn_norm, (T*)s.u, Tn, d, c.rms_eps, st));
    void *kc, *vc;
    kv_layer(m, kv, layer, &kc, &vc);
    // q, k and v in one product: the columns of W_k and W_v follow those of W_q;
    // RoPE and the cache write run in its split-K epilogue when it has one
    RopeEpi re{s.q, kc, vc, B, n, pos0, kv->cap, c.n_heads, c.n_kv_heads, dh, c.rope_on,
               c.rope_theta, false};
    DG_TRY(linear<T>(s.u, Tn, d, L.wq, qkvw, s.qkv, qkvw, dg::EPI_STORE_F32, s, st, nullptr,
                     nullptr, 0, 0, L.wk, c.n_heads * dh, L.wv, (c.n_heads + c.n_kv_heads) * dh,
                     &re));
    if (!re.done)
        DG_HIP(dg::rope_kv<T>(s.qkv, (T*)s.q, (T*)kc, (T*)vc, B, n, pos0, kv->cap, c.n_heads,
                              c.n_kv_heads, dh, c.rope_on, c.rope_theta, st));
    dg::AttnArgs a;
    a.q = s.q;
    a.kc = kc;
    a.vc = vc;
    a.out = s.ao;
    a.part_o = s.part_o;
    a.part_ml = s.part_ml;
    a.B = B;
    a.n = n;
    a.pos0 = pos0;
    a.cap = kv->cap;
    a.Hq = c.n_heads;
    a.Hkv = c.n_kv_heads;
    a.dh = dh;
    a.kv_len = pos0 + n;
    a.causal = causal;
    a.halt = s.halt;
    // the split merge handles heads of 64 or more dimensions
    const int max_splits =
        dh < 64 ? 1 : std::max(1, std::max(kAttnPartRows, 8 * B * c.canvas) / Tn);
    a.splits = dg::attention_splits(B, n, c.n_heads, c.n_kv_heads, a.kv_len, causal, max_splits,
                                    &a.split_len, dh, sizeof(T) == 2);
    DG_HIP(timed(DG_TIMER_ATTENTION, st, [&] { return dg::attention<T>(a, st); }));
    // (moe_norm: the MoE half's RMSNorm runs in this product's epilogue when it can)
    DG_TRY(linear<T>(s.ao, Tn, c.n_heads * dh, L.wo, d, h, d, dg::EPI_ADD_F32, s, st, nullptr,
                     nullptr, 0, 0, nullptr, 0, nullptr, 0, nullptr, moe_norm));
    return DG_OK;
}

// the MoE half's RMSNorm outputs, as moe_half's own rmsnorm call writes them
template <typename T>
AddNormEpi moe_norm_epi(const dg_model* m, int layer, const Scratch& s) {
    const bool b = sizeof(T) == 2;
    return AddNormEpi{m->layers[layer].moe_norm, s.u, b ? s.u32 : nullptr, b ? s.u8 : nullptr,
                      b ? s.u8s : nullptr, m->c.rms_eps, false};
}

// next_norm: the next layer's attention RMSNorm weight, to fuse that norm into
// the combine (then *normed is set and s.u holds its output)
template <typename T>
dg_status moe_half(dg_model* m, int layer, int Tn, float* h, Scratch& s, hipStream_t st,
                   const float* next_norm = nullptr, bool* normed = nullptr,
                   bool moe_normed = false) {
    const dg_config& c = m->c;
    const dg_layer_weights& L = m->layers[layer];
    // canvas-sized batches: the router product runs inside the routing kernel
    const bool fused_router = sizeof(T) == 2 && dg::router_fused_ok(Tn, c.d_model, c.n_experts);
    if (sizeof(T) == 2) {
        // The route is an integer decision taken from float logits: compute
        // them from the fp32 normalised activations (written by the same
        // kernel as the bf16 ones) and the bf16 router weights widened to
        // fp32 on load, so bf16 rounding of the activations cannot flip it.
        if (!moe_normed)
            DG_HIP(dg::rmsnorm<T>(h, L.moe_norm, (T*)s.u, Tn, c.d_model, c.rms_eps, st, s.u32,
                                  s.u8, s.u8s));
        if (!fused_router)
            DG_TRY(linear<float>(s.u32, Tn, c.d_model, L.w_router, c.n_experts, s.z, c.n_experts,
                                 dg::EPI_STORE_F32, s, st, nullptr, nullptr, 0, 1));
    } else {
        if (!moe_normed) DG_HIP(dg::rmsnorm<T>(h, L.moe_norm, (T*)s.u, Tn, c.d_model, c.rms_eps, st));
        DG_TRY(linear<T>(s.u, Tn, c.d_model, L.w_router, c.n_experts, s.z, c.n_experts,
                         dg::EPI_STORE_F32, s, st));
    }
    dg::MoeArgs a;
    a.T = Tn;
    a.d = c.d_model;
    a.E = c.n_experts;
    a.k = c.top_k;
    a.F = c.d_ff;
    a.z = s.z;
    a.route = s.route;
    a.gates = s.gates;
    a.counts = s.counts;
    a.offsets = s.offsets;
    a.order = s.order;
    if (c.expert_dtype == DG_FP8_E4M3) {
        a.f8 = 1;
        a.s_gate = L.s_gate;
        a.s_up = L.s_up;
        a.s_down = L.s_down;
    } else if (c.expert_dtype == DG_MXFP4) {
        a.f4 = 1;
        a.x_gate = L.x_gate;
        a.x_up = L.x_up;
        a.x_down = L.x_down;
    }
    a.perm_tok = s.perm_tok;
    a.slot_of = s.slot_of;
    a.u = s.u;
    a.w_gate = L.w_gate;
    a.w_up = L.w_up;
    a.w_down = L.w_down;
    a.act = s.act;
    a.u8 = s.u8;
    a.u8s = s.u8s;
    a.act8 = s.act8;
    a.act8s = s.act8s;
    a.work = s.work;
    a.items = s.items;
    a.y = s.y;
    a.h = h;
    a.k_rotate = 1;
    a.halt = s.halt;
    if (fused_router) {
        a.router_u = s.u32;
        a.router_w = L.w_router;
    }
    DG_HIP(dg::moe_route(a, st));
    DG_HIP(timed(DG_TIMER_MOE_GATEUP, st, [&] { return dg::moe_gateup<T>(a, st); }));
    DG_HIP(timed(DG_TIMER_MOE_DOWN, st, [&] { return dg::moe_down<T>(a, st); }));
    if (normed) *normed = false;
    if (next_norm && dg::moe_combine_norm_ok(c.top_k)) {
        DG_HIP(dg::moe_combine_norm<T>(a, next_norm, (T*)s.u, c.rms_eps, st));
        if (normed) *normed = true;
    } else {
        DG_HIP(dg::moe_combine(a, st));
    }
    return DG_OK;
}

// h[B*N][d] = E[canvas] + (softmax(prev) E) W_sc^T
template <typename T>
dg_status stage_input(dg_model* m, int B, const int32_t* canvas, const float* prev_logits,
                      const float* prev_stats, float* h, Scratch& s, hipStream_t st) {
    const dg_config& c = m->c;
    const int Tn = B * c.canvas;
    if (!prev_logits) {
        DG_HIP(dg::embed_rows<T>((const T*)m->embed, c.vocab, canvas, c.canvas, c.canvas, B, h, c.d_model,
                                 st));
        return DG_OK;
    }
    if (s.topk > 0) {
        // the previous distribution truncated to each position's top-k:
        // candidates and weights from the sampler (block loop) or from the
        // same selection run on the previous logits, then the gathered sum
        if (!s.topk_ready) {
            dg::SampleArgs a;
            a.B = 1;
            a.N = Tn;
            a.V = c.vocab;
            a.top_k = s.topk;
            a.logits = prev_logits;
            a.stop = s.zero;
            a.tk_idx = s.tk_idx;
            a.tk_p = s.tk_p;
            a.list_only = 1;
            DG_HIP(dg::fill_i32(s.zero, 0, 1, st));
            DG_HIP(dg::sample_update(a, st));
        }
        DG_HIP(dg::selfcond_topk<T>((const T*)m->embed, c.d_model, s.tk_idx, s.tk_p, s.topk, Tn,
                                    (T*)s.sc_s, st));
        DG_TRY(linear<T>(s.sc_s, Tn, c.d_model, m->w_sc, c.d_model, h, c.d_model,
                         dg::EPI_EMBED_ADD, s, st, m->embed, canvas, c.vocab));
        return DG_OK;
    }
    if (!m->embed_t) return fail(DG_ERR_ARG, "self-conditioning needs weights.embed_t");
    const int splits = sc_splits(m, Tn);
    dg::GemmArgs g;
    g.M = Tn;
    g.N = c.d_model;
    g.K = c.vocab;
    g.A = prev_logits;
    g.lda = c.vocab;
    g.a_stats = prev_stats;
    g.B = m->embed_t;
    g.ldb = c.vocab;
    g.C = s.sc_part;
    g.ldc = c.d_model;
    // k-ranges in whole 128-element steps (the bf16 ring kernel walks four
    // 32-element stages at a time)
    g.k_split = cdiv(cdiv(c.vocab, splits), 128) * 128;
    const int used = cdiv(c.vocab, g.k_split);
    if (sizeof(T) == 2) {
        // probabilities once in bf16, then the streaming product over the
        // vocabulary split into `used` k-ranges (column tiles of a range on
        // one XCD)
        // unnormalised probabilities once in bf16 (the 1 / sum factor is
        // applied in the split-K reduction); in the block loop the sampler
        // has already written them
        if (!s.probs_ready)
            DG_HIP(dg::selfcond_probs(prev_logits, prev_stats, (uint16_t*)s.probs, Tn, c.vocab,
                                      s.halt, s.probs_tiled, st));
        g.A = s.probs;
        g.a_tiled = s.probs_tiled ? 2 : 0;
        g.b_tiled = m->blocked ? 1 : 0;
        g.xcd_group = (used % 8 == 0 && cdiv(c.d_model, 256) > 1) ? 1 : 0;
        g.k_rotate = 1;
        g.halt = s.halt;
        DG_HIP(timed(DG_TIMER_SELFCOND_GEMM, st,
                     [&] { return dg::gemm_tn<T>(g, 0, dg::EPI_SPLITK, used, st); }));
    } else {
        DG_HIP(timed(DG_TIMER_SELFCOND_GEMM, st,
                     [&] { return dg::gemm_tn<T>(g, 1, dg::EPI_SPLITK, used, st); }));
    }
    DG_HIP(dg::splitk_reduce<T>(s.sc_part, (T*)s.sc_s, used, Tn, c.d_model, st,
                                sizeof(T) == 2 ? prev_stats : nullptr));
    DG_TRY(linear<T>(s.sc_s, Tn, c.d_model, m->w_sc, c.d_model, h, c.d_model, dg::EPI_EMBED_ADD, s,
                     st, m->embed, canvas, c.vocab));
    return DG_OK;
}

template <typename T>
dg_status stage_head(dg_model* m, int Tn, const float* h, float* logits, Scratch& s,
                     hipStream_t st) {
    const dg_config& c = m->c;
    dg::GemmArgs g;
    g.M = Tn;
    g.N = c.vocab;
    g.K = c.d_model;
    g.B = m->embed;
    g.ldb = c.d_model;
    g.C = logits;
    g.ldc = c.vocab;
    g.k_split = c.d_model;
    g.k_rotate = 1;
    g.halt = s.halt;
    if (m->blocked && m->embed_head && Tn <= s.ut_rows) {
        // both operands in the blocked layout: each stage of a tile is one
        // contiguous 16 KiB block of E and of the normalised rows
        DG_HIP(dg::rmsnorm_tiled(h, m->final_norm, (uint16_t*)s.ut, Tn, c.d_model, c.rms_eps, st));
        g.A = s.ut;
        g.B = m->embed_head;
        g.a_tiled = g.b_tiled = 1;
        if (s.want_rowmax) g.rowmax = s.tmax;
    } else {
        DG_HIP(dg::rmsnorm<T>(h, m->final_norm, (T*)s.u, Tn, c.d_model, c.rms_eps, st));
        g.A = s.u;
        g.lda = c.d_model;
    }
    if (g.a_tiled && dg::gemm_decode_ok(g))
        DG_HIP(timed(DG_TIMER_HEAD_GEMM, st, [&] { return dg::gemm_decode(g, st); }));
    else
        DG_HIP(timed(DG_TIMER_HEAD_GEMM, st,
                     [&] { return dg::gemm_tn<T>(g, 0, dg::EPI_STORE_F32, 1, st); }));
    return DG_OK;
}

template <typename T>
dg_status denoise(dg_model* m, dg_kv* kv, int B, const int32_t* canvas, const float* prev,
                  const float* prev_stats, float* logits, Scratch& s, hipStream_t st) {
    const dg_config& c = m->c;
    const int Tn = B * c.canvas;
    DG_TRY(stage_input<T>(m, B, canvas, prev, prev_stats, s.h, s, st));
    bool normed = false;
    for (int l = 0; l < c.n_layers; ++l) {
        AddNormEpi mn = moe_norm_epi<T>(m, l, s);
        DG_TRY(attn_half<T>(m, kv, l, B, c.canvas, kv->len, 0, s.h, s, st, normed, &mn));
        DG_TRY(moe_half<T>(m, l, Tn, s.h, s, st, next_attn_norm(m, l), &normed, mn.done));
    }
    return stage_head<T>(m, Tn, s.h, logits, s, st);
}

template <typename T>
dg_status encode(dg_model* m, dg_kv* kv, int B, const int32_t* tokens, int P, Scratch& s,
                 hipStream_t st) {
    const dg_config& c = m->c;
    const int chunk = std::max(1, token_budget(m, B) / B);
    for (int c0 = 0; c0 < P; c0 += chunk) {
        const int n = std::min(chunk, P - c0);
        const int pos0 = kv->len + c0;
        DG_HIP(dg::embed_rows<T>((const T*)m->embed, c.vocab, tokens + c0, P, n, B, s.h, c.d_model, st));
        bool normed = false;
        for (int l = 0; l < c.n_layers; ++l) {
            const bool last = l + 1 == c.n_layers;   // its MoE half is not needed
            AddNormEpi mn = moe_norm_epi<T>(m, l, s);
            DG_TRY(attn_half<T>(m, kv, l, B, n, pos0, 1, s.h, s, st, normed, last ? nullptr : &mn));
            if (!last)
                DG_TRY(moe_half<T>(m, l, B * n, s.h, s, st, next_attn_norm(m, l), &normed,
                                   mn.done));
        }
    }
    kv->len += P;
    return DG_OK;
}

// Retained autoregressive mode: one token per sequence at position kv->len
// (token b at tokens[b * ld]), causal attention over the cache in every
// layer, every layer's MoE, then the head on the new tokens.
template <typename T>
dg_status ar_decode(dg_model* m, dg_kv* kv, int B, const int32_t* tokens, int ld, float* logits,
                    Scratch& s, hipStream_t st) {
    const dg_config& c = m->c;
    const int pos0 = kv->len;
    DG_HIP(dg::embed_rows<T>((const T*)m->embed, c.vocab, tokens, ld, 1, B, s.h, c.d_model, st));
    bool normed = false;
    for (int l = 0; l < c.n_layers; ++l) {
        AddNormEpi mn = moe_norm_epi<T>(m, l, s);
        DG_TRY(attn_half<T>(m, kv, l, B, 1, pos0, 1, s.h, s, st, normed, &mn));
        DG_TRY(moe_half<T>(m, l, B, s.h, s, st, next_attn_norm(m, l), &normed, mn.done));
    }
    kv->len += 1;
    return stage_head<T>(m, B, s.h, logits, s, st);
}

dg_status check_model(const dg_model* m) {
    if (!m) return fail(DG_ERR_ARG, "model is NULL");
    return DG_OK;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

}  // namespace

// ---- dg_sample_update_static: the sampler's scratch in a static device array
//
// For callers that cannot allocate device memory.  The scratch of
// dg_sample_update (drawn tokens, renoise tokens and the new argmax, one
// int32 each per row, every one written by the row pass before the canvas
// pass reads it, so nothing needs clearing) lives in `scratch`, one copy per
// GPU for the life of the process.  Host code never passes `scratch` itself
// (that is a host-side stand-in, not a device address): the device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address goes to the kernels.
constexpr int kStaticSamplerRows = 65536;   // batch * canvas at most
constexpr size_t kStaticSamplerBytes =
    3 * (((size_t)kStaticSamplerRows * 4 + 255) & ~(size_t)255) + 256;
static __device__ __align__(256) unsigned char scratch[kStaticSamplerBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's `scratch` (looked up on first use).
dg_status static_scratch(void** out) {
    int dev = 0;
    DG_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_UNSUPPORTED, "device %d", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        DG_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return fail(DG_ERR_HIP, "no device address for the sampler scratch");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DG_OK;
}
}  // namespace

// ======================================================================= API

extern "C" {

const char* dg_status_string(dg_status s) {
    switch (s) {
        case DG_OK: return "ok";
        case DG_ERR_ARG: return "invalid argument";
        case DG_ERR_SHAPE: return "unsupported or inconsistent shape";
        case DG_ERR_DTYPE: return "unknown dtype";
        case DG_ERR_CAPACITY: return "capacity exceeded";
        case DG_ERR_NONFINITE: return "non-finite values";
        case DG_ERR_HIP: return "HIP runtime error";
        case DG_ERR_UNSUPPORTED: return "unsupported";
    }
    return "unknown status";
}

const char* dg_last_error(void) { return g_err.c_str(); }

dg_status dg_model_create(const dg_config* cfg, const dg_weights* w, dg_model** out) {
    if (!cfg || !w || !out) return fail(DG_ERR_ARG, "NULL argument");
    *out = nullptr;
    const dg_config& c = *cfg;
    if (c.dtype != DG_F32 && c.dtype != DG_BF16) return fail(DG_ERR_DTYPE, "dtype %d", c.dtype);
    if (c.n_layers < 1 || c.d_model < 64 || c.d_model % 64 != 0)
        return fail(DG_ERR_SHAPE, "n_layers >= 1 and d_model a multiple of 64 required");
    if (c.n_heads < 1 || c.n_kv_heads < 1 || c.n_heads % c.n_kv_heads != 0)
        return fail(DG_ERR_SHAPE, "n_heads must be a positive multiple of n_kv_heads");
    const bool dh_ok = c.head_dim == 64 || c.head_dim == 128 ||
                       (c.head_dim == 256 && c.dtype == DG_BF16);
    if (!dh_ok) return fail(DG_ERR_SHAPE, "head_dim %d unsupported (64, 128; 256 in bf16)",
                            c.head_dim);
    if (c.n_experts < 1 || c.n_experts > 256 || c.top_k < 1 || c.top_k > 16 ||
        c.top_k > c.n_experts)
        return fail(DG_ERR_SHAPE, "need 1 <= top_k <= min(n_experts, 16), n_experts <= 256");
    if (c.d_ff < 32 || c.d_ff % 32 != 0) return fail(DG_ERR_SHAPE, "d_ff must be a multiple of 32");
    if (c.vocab < 8 || c.vocab > 524288 || c.vocab % 8 != 0)
        return fail(DG_ERR_SHAPE, "vocab must be a multiple of 8 in [8, 524288]");
    if (c.canvas < 1 || c.canvas > 1024) return fail(DG_ERR_SHAPE, "canvas must be in [1, 1024]");
    if (!(c.rms_eps >= 0.f) || (c.rope_on && !(c.rope_theta > 0.f)))
        return fail(DG_ERR_ARG, "rms_eps >= 0 and rope_theta > 0 required");
    if (!w->embed || !w->w_sc || !w->layers) return fail(DG_ERR_ARG, "missing weights");
    for (int l = 0; l < c.n_layers; ++l) {
        const dg_layer_weights& L = w->layers[l];
        if (!L.wq || !L.wk || !L.wv || !L.wo || !L.w_router || !L.w_gate || !L.w_up || !L.w_down)
            return fail(DG_ERR_ARG, "missing weights in layer %d", l);
    }
    if (c.expert_dtype != 0 && c.expert_dtype != c.dtype && c.expert_dtype != DG_FP8_E4M3 &&
        c.expert_dtype != DG_MXFP4)
        return fail(DG_ERR_DTYPE, "expert_dtype %d", c.expert_dtype);
    const bool quantised_experts = c.expert_dtype == DG_MXFP4 || c.expert_dtype == DG_FP8_E4M3;
    if (quantised_experts && (c.dtype != DG_BF16 || c.d_model % 128 || c.d_ff % 128))
        // the block-scaled MFMA kernels take 128 k per step, 64 gate/up
        // features and 128 down rows per workgroup
        return fail(DG_ERR_UNSUPPORTED,
                    "quantised experts need a bf16 model with d_model and d_ff multiples of 128");
    if (c.expert_dtype == DG_MXFP4) {
        for (int l = 0; l < c.n_layers; ++l) {
            const dg_layer_weights& L = w->layers[l];
            if (!L.x_gate || !L.x_up || !L.x_down)
                return fail(DG_ERR_ARG, "MXFP4 experts need x_gate, x_up and x_down (layer %d)", l);
        }
    }
    if (c.expert_dtype == DG_FP8_E4M3) {
        for (int l = 0; l < c.n_layers; ++l) {
            const dg_layer_weights& L = w->layers[l];
            if (!L.s_gate || !L.s_up || !L.s_down)
                return fail(DG_ERR_ARG, "FP8 experts need s_gate, s_up and s_down (layer %d)", l);
        }
    }
    dg_model* m = new dg_model;
    m->c = c;
    m->embed = w->embed;
    m->embed_t = w->embed_t;
    m->embed_head = w->embed_head;
    m->blocked = c.dtype == DG_BF16 && c.d_model % 256 == 0 && c.vocab % 128 == 0;
    m->w_sc = w->w_sc;
    m->final_norm = w->final_norm;
    m->layers.assign(w->layers, w->layers + c.n_layers);
    // the block loop's stop-flag slots and their events, freed with the
    // model.  Without a usable device they stay absent: creation still
    // succeeds (validation needs no GPU) and the block loop reports it.
    bool loop_ok = true;
    for (hipEvent_t& e : m->flag_ev)
        if (loop_ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
            e = nullptr;
            loop_ok = false;
        }
    if (loop_ok &&
        hipHostMalloc((void**)&m->hflags, 2 * (size_t)DG_MAX_LOOP_BATCH * sizeof(int32_t)) ==
            hipSuccess)
        m->hflags_cap = DG_MAX_LOOP_BATCH;
    else
        m->hflags = nullptr;
    (void)hipGetLastError();   // a failure here is reported by the block loop
    *out = m;
    return DG_OK;
}

void dg_model_destroy(dg_model* m) { delete m; }

dg_status dg_quantize_fp8(const void* d_src, int32_t src_dtype, int64_t rows, int32_t cols,
                          void* d_q, float* d_scale, void* stream) {
    if (!d_src || !d_q || !d_scale) return fail(DG_ERR_ARG, "NULL pointer");
    if (rows < 16 || cols < 128 || rows % 16 || cols % 128 || rows > 0x7FFFFFFF)
        return fail(DG_ERR_ARG, "bad sizes (rows a multiple of 16, cols of 128)");
    if (src_dtype == DG_BF16)
        DG_HIP(dg::quantize_fp8<bf16_t>((const bf16_t*)d_src, (long)rows, cols, (uint8_t*)d_q,
                                        d_scale, as_stream(stream)));
    else if (src_dtype == DG_F32)
        DG_HIP(dg::quantize_fp8<float>((const float*)d_src, (long)rows, cols, (uint8_t*)d_q,
                                       d_scale, as_stream(stream)));
    else
        return fail(DG_ERR_DTYPE, "src_dtype %d", src_dtype);
    return DG_OK;
}

dg_status dg_quantize_mxfp4(const void* d_src, int32_t src_dtype, int64_t rows, int32_t cols,
                            void* d_codes, uint8_t* d_scales, void* stream) {
    if (!d_src || !d_codes || !d_scales) return fail(DG_ERR_ARG, "NULL pointer");
    if (rows < 16 || cols < 128 || rows % 16 || cols % 128 || rows > 0x7FFFFFFF)
        return fail(DG_ERR_ARG, "bad sizes (rows a multiple of 16, cols of 128)");
    if (src_dtype == DG_BF16)
        DG_HIP(dg::quantize_mxfp4<bf16_t>((const bf16_t*)d_src, (long)rows, cols,
                                          (uint8_t*)d_codes, d_scales, as_stream(stream)));
    else if (src_dtype == DG_F32)
        DG_HIP(dg::quantize_mxfp4<float>((const float*)d_src, (long)rows, cols, (uint8_t*)d_codes,
                                         d_scales, as_stream(stream)));
    else
        return fail(DG_ERR_DTYPE, "src_dtype %d", src_dtype);
    return DG_OK;
}

dg_status dg_embed_transpose(const dg_model* m, const void* d_embed, void* d_out, void* stream) {
    DG_TRY(check_model(m));
    if (!d_embed || !d_out) return fail(DG_ERR_ARG, "NULL pointer");
    if (m->blocked)
        DG_HIP(dg::embed_tile((const uint16_t*)d_embed, m->c.vocab, m->c.d_model, 1,
                              (uint16_t*)d_out, as_stream(stream)));
    else if (m->c.dtype == DG_BF16)
        DG_HIP(dg::transpose<bf16_t>((const bf16_t*)d_embed, (bf16_t*)d_out,
                                         m->c.vocab, m->c.d_model, as_stream(stream)));
    else
        DG_HIP(dg::transpose<float>((const float*)d_embed, (float*)d_out, m->c.vocab,
                                    m->c.d_model, as_stream(stream)));
    return DG_OK;
}

dg_status dg_embed_head_bytes(const dg_model* m, size_t* bytes) {
    DG_TRY(check_model(m));
    if (!bytes) return fail(DG_ERR_ARG, "NULL pointer");
    *bytes = m->blocked ? (size_t)cdiv(m->c.vocab, 256) * 256 * m->c.d_model * 2 : 0;
    return DG_OK;
}

dg_status dg_embed_head(const dg_model* m, const void* d_embed, void* d_out, void* stream) {
    DG_TRY(check_model(m));
    if (!d_embed || !d_out) return fail(DG_ERR_ARG, "NULL pointer");
    if (!m->blocked) return fail(DG_ERR_UNSUPPORTED, "this model's head reads embed directly");
    DG_HIP(dg::embed_tile((const uint16_t*)d_embed, m->c.vocab, m->c.d_model, 0, (uint16_t*)d_out,
                          as_stream(stream)));
    return DG_OK;
}

dg_status dg_kv_bytes(const dg_model* m, int32_t batch, int32_t capacity, size_t* bytes) {
    DG_TRY(check_model(m));
    if (!bytes || batch < 1 || capacity < 1) return fail(DG_ERR_ARG, "bad kv size request");
    const dg_config& c = m->c;
    *bytes = 2 * (size_t)c.n_layers * batch * c.n_kv_heads * capacity * c.head_dim *
             elt_size(c.dtype);
    return DG_OK;
}

dg_status dg_kv_create(const dg_model* m, int32_t batch, int32_t capacity, void* d_buf,
                       dg_kv** out) {
    DG_TRY(check_model(m));
    if (!d_buf || !out || batch < 1 || capacity < 1) return fail(DG_ERR_ARG, "bad kv arguments");
    dg_kv* kv = new dg_kv;
    kv->B = batch;
    kv->cap = capacity;
    kv->len = 0;
    kv->buf = d_buf;
    *out = kv;
    return DG_OK;
}

void dg_kv_destroy(dg_kv* kv) { delete kv; }

dg_status dg_kv_length(const dg_kv* kv, int32_t* len) {
    if (!kv || !len) return fail(DG_ERR_ARG, "NULL argument");
    *len = kv->len;
    return DG_OK;
}

dg_status dg_kv_set_length(dg_kv* kv, int32_t len) {
    if (!kv) return fail(DG_ERR_ARG, "NULL argument");
    if (len < 0 || len > kv->cap) return fail(DG_ERR_CAPACITY, "length %d outside [0, %d]", len,
                                              kv->cap);
    kv->len = len;
    return DG_OK;
}

dg_status dg_workspace_bytes(const dg_model* m, int32_t batch, size_t* bytes) {
    DG_TRY(check_model(m));
    if (!bytes || batch < 1) return fail(DG_ERR_ARG, "bad workspace request");
    Carver cv(nullptr, 0);
    Scratch s;
    carve_scratch(cv, m, batch, s);
    *bytes = cv.off + 256;
    return DG_OK;
}

dg_status dg_sampler_workspace_bytes(int32_t batch, int32_t canvas, size_t* bytes) {
    if (!bytes || batch < 1 || canvas < 1) return fail(DG_ERR_ARG, "bad sampler workspace request");
    *bytes = 3 * (((size_t)batch * canvas * 4 + 255) & ~(size_t)255) + 256;
    return DG_OK;
}

dg_status dg_encode_prompt(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_tokens,
                           int32_t n_tokens, void* d_ws, size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!kv || !d_tokens || n_tokens < 0) return fail(DG_ERR_ARG, "bad encode arguments");
    if (batch != kv->B) return fail(DG_ERR_SHAPE, "batch %d != cache batch %d", batch, kv->B);
    if (kv->len + n_tokens > kv->cap)
        return fail(DG_ERR_CAPACITY, "len %d + %d tokens exceeds capacity %d", kv->len, n_tokens,
                    kv->cap);
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, batch, d_ws, ws_bytes, s, cv));
    if (n_tokens == 0) return DG_OK;
    if (m->c.dtype == DG_BF16)
        return encode<bf16_t>(m, kv, batch, d_tokens, n_tokens, s, as_stream(stream));
    return encode<float>(m, kv, batch, d_tokens, n_tokens, s, as_stream(stream));
}

dg_status dg_commit_block(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_block,
                          void* d_ws, size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    return dg_encode_prompt(m, kv, batch, d_block, m->c.canvas, d_ws, ws_bytes, stream);
}

dg_status dg_ar_decode_step(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_tokens,
                            float* d_logits, void* d_ws, size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!kv || !d_tokens || !d_logits) return fail(DG_ERR_ARG, "NULL argument");
    if (batch != kv->B) return fail(DG_ERR_SHAPE, "batch %d != cache batch %d", batch, kv->B);
    if (kv->len + 1 > kv->cap)
        return fail(DG_ERR_CAPACITY, "cache of capacity %d is full", kv->cap);
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, batch, d_ws, ws_bytes, s, cv));
    if (m->c.dtype == DG_BF16)
        return ar_decode<bf16_t>(m, kv, batch, d_tokens, 1, d_logits, s, as_stream(stream));
    return ar_decode<float>(m, kv, batch, d_tokens, 1, d_logits, s, as_stream(stream));
}

dg_status dg_argmax_rows(int32_t rows, int32_t vocab, const float* d_logits, int32_t* d_out,
                         void* stream) {
    if (rows < 0 || vocab < 1 || (rows > 0 && (!d_logits || !d_out)))
        return fail(DG_ERR_ARG, "bad argmax arguments");
    if ((uintptr_t)d_logits & 15) return fail(DG_ERR_ARG, "logits must be 16-byte aligned");
    DG_HIP(dg::argmax_rows(d_logits, rows, vocab, d_out, 1, as_stream(stream)));
    return DG_OK;
}

dg_status dg_ar_generate(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_first,
                         int32_t n_new, int32_t* d_out, float* d_logits, void* d_ws,
                         size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!kv || !d_first || !d_out || !d_logits || n_new < 0)
        return fail(DG_ERR_ARG, "bad generate arguments");
    if (batch != kv->B) return fail(DG_ERR_SHAPE, "batch %d != cache batch %d", batch, kv->B);
    if (kv->len + n_new > kv->cap)
        return fail(DG_ERR_CAPACITY, "len %d + %d tokens exceeds capacity %d", kv->len, n_new,
                    kv->cap);
    if ((uintptr_t)d_logits & 15) return fail(DG_ERR_ARG, "logits must be 16-byte aligned");
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, batch, d_ws, ws_bytes, s, cv));
    const dg_config& c = m->c;
    hipStream_t st = as_stream(stream);
    // the head's slab maxima make the greedy choice a read of 16 KB + one
    // slab per row (blocked bf16 models); otherwise one pass over the row
    const bool slabs = m->blocked && m->embed_head && batch <= s.ut_rows && c.vocab % 64 == 0;
    s.want_rowmax = slabs;
    for (int t = 0; t < n_new; ++t) {
        const int32_t* tok = t == 0 ? d_first : d_out + (t - 1);
        const int ld = t == 0 ? 1 : n_new;
        if (c.dtype == DG_BF16)
            DG_TRY(ar_decode<bf16_t>(m, kv, batch, tok, ld, d_logits, s, st));
        else
            DG_TRY(ar_decode<float>(m, kv, batch, tok, ld, d_logits, s, st));
        if (slabs)
            DG_HIP(dg::argmax_slabs(d_logits, s.tmax, batch, c.vocab, d_out + t, n_new, st));
        else
            DG_HIP(dg::argmax_rows(d_logits, batch, c.vocab, d_out + t, n_new, st));
    }
    return DG_OK;
}

dg_status dg_corrupt(uint64_t seed, int32_t step, int32_t batch, int32_t canvas, int32_t vocab,
                     const float* d_rate, const int32_t* d_clean, int32_t* d_out, void* stream) {
    if (batch < 0 || canvas < 0 || vocab < 1 ||
        ((long)batch * canvas > 0 && (!d_rate || !d_clean || !d_out)))
        return fail(DG_ERR_ARG, "bad corruption arguments");
    DG_HIP(dg::corrupt(seed, step, batch, canvas, vocab, d_rate, d_clean, d_out,
                       as_stream(stream)));
    return DG_OK;
}

static dg_status xent_impl(int32_t rows, int32_t vocab, const float* d_logits,
                           const int32_t* d_target, float* d_loss, float* d_mean,
                           hipStream_t st) {
    dg::SampleArgs a;
    a.B = 1;
    a.N = rows;
    a.V = vocab;
    a.inv_t = 1.0f;
    a.logits = d_logits;
    a.stats_only = 1;
    a.target = d_target;
    a.loss = d_loss;
    DG_HIP(timed(DG_TIMER_SAMPLER, st, [&] { return dg::sample_update(a, st); }));
    if (d_mean) DG_HIP(dg::mean_seq(d_loss, rows, d_mean, st));
    return DG_OK;
}

dg_status dg_xent(int32_t rows, int32_t vocab, const float* d_logits, const int32_t* d_target,
                  float* d_loss, float* d_mean, void* stream) {
    if (rows < 1 || vocab < 1 || !d_logits || !d_target || !d_loss)
        return fail(DG_ERR_ARG, "bad cross-entropy arguments");
    if (vocab > (1 << 19)) return fail(DG_ERR_ARG, "vocab %d above 2^19", vocab);
    return xent_impl(rows, vocab, d_logits, d_target, d_loss, d_mean, as_stream(stream));
}

dg_status dg_train_forward(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_clean,
                           const float* d_rate, uint64_t seed, int32_t step, int32_t* d_corrupted,
                           float* d_logits, float* d_loss, float* d_mean, void* d_ws,
                           size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!kv || !d_clean || !d_rate || !d_corrupted || !d_logits || !d_loss)
        return fail(DG_ERR_ARG, "NULL argument");
    if (batch != kv->B) return fail(DG_ERR_SHAPE, "batch %d != cache batch %d", batch, kv->B);
    if (kv->len + m->c.canvas > kv->cap)
        return fail(DG_ERR_CAPACITY, "cache needs len %d + canvas %d <= capacity %d", kv->len,
                    m->c.canvas, kv->cap);
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, batch, d_ws, ws_bytes, s, cv));
    const dg_config& c = m->c;
    hipStream_t st = as_stream(stream);
    DG_HIP(dg::corrupt(seed, step, batch, c.canvas, c.vocab, d_rate, d_clean, d_corrupted, st));
    if (c.dtype == DG_BF16)
        DG_TRY(denoise<bf16_t>(m, kv, batch, d_corrupted, nullptr, nullptr, d_logits, s, st));
    else
        DG_TRY(denoise<float>(m, kv, batch, d_corrupted, nullptr, nullptr, d_logits, s, st));
    return xent_impl(batch * c.canvas, c.vocab, d_logits, d_clean, d_loss, d_mean, st);
}

dg_status dg_denoise_step_topk(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_canvas,
                               const float* d_prev_logits, const float* d_prev_stats,
                               int32_t top_k, float* d_logits, void* d_ws, size_t ws_bytes,
                               void* stream) {
    if (top_k == 0)
        return dg_denoise_step(m, kv, batch, d_canvas, d_prev_logits, d_prev_stats, d_logits,
                               d_ws, ws_bytes, stream);
    DG_TRY(check_model(m));
    if (!kv || !d_canvas || !d_logits || !d_prev_logits) return fail(DG_ERR_ARG, "NULL argument");
    if (top_k < 0 || top_k > dg::kTopKMax || top_k > m->c.vocab)
        return fail(DG_ERR_ARG, "top_k %d outside [0, min(64, vocab)]", top_k);
    if (batch != kv->B) return fail(DG_ERR_SHAPE, "batch %d != cache batch %d", batch, kv->B);
    if (kv->len + m->c.canvas > kv->cap)
        return fail(DG_ERR_CAPACITY, "cache needs len %d + canvas %d <= capacity %d", kv->len,
                    m->c.canvas, kv->cap);
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, batch, d_ws, ws_bytes, s, cv));
    s.topk = top_k;
    if (m->c.dtype == DG_BF16)
        return denoise<bf16_t>(m, kv, batch, d_canvas, d_prev_logits, d_prev_stats, d_logits,
                               s, as_stream(stream));
    return denoise<float>(m, kv, batch, d_canvas, d_prev_logits, d_prev_stats, d_logits, s,
                          as_stream(stream));
}

dg_status dg_denoise_step(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_canvas,
                          const float* d_prev_logits, const float* d_prev_stats, float* d_logits,
                          void* d_ws, size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!kv || !d_canvas || !d_logits) return fail(DG_ERR_ARG, "NULL argument");
    if ((d_prev_logits == nullptr) != (d_prev_stats == nullptr))
        return fail(DG_ERR_ARG, "prev_logits and prev_stats must both be set or both NULL");
    if (batch != kv->B) return fail(DG_ERR_SHAPE, "batch %d != cache batch %d", batch, kv->B);
    if (kv->len + m->c.canvas > kv->cap)
        return fail(DG_ERR_CAPACITY, "cache needs len %d + canvas %d <= capacity %d", kv->len,
                    m->c.canvas, kv->cap);
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, batch, d_ws, ws_bytes, s, cv));
    if (m->c.dtype == DG_BF16)
        return denoise<bf16_t>(m, kv, batch, d_canvas, d_prev_logits, d_prev_stats, d_logits,
                                   s, as_stream(stream));
    return denoise<float>(m, kv, batch, d_canvas, d_prev_logits, d_prev_stats, d_logits, s,
                          as_stream(stream));
}

static dg_status sample_impl(const dg_sampler_params* p, int32_t step, int32_t batch,
                             int32_t canvas, int32_t vocab, const float* d_logits,
                             int32_t* d_canvas, int32_t* d_argmax, uint8_t* d_lock,
                             float* d_stats, int32_t* d_stop, void* d_ws, size_t ws_bytes,
                             hipStream_t st, int32_t* nstop = nullptr,
                             int32_t* halt = nullptr, const float* rowmax = nullptr,
                             void* probs = nullptr, int probs_tiled = 1,
                             int32_t* host_stop = nullptr, int32_t* tk_idx = nullptr,
                             float* tk_p = nullptr, bool untimed = false,
                             float* trace = nullptr) {
    if (!p || !d_logits || !d_canvas || !d_argmax || !d_lock || !d_stats || !d_stop || !d_ws)
        return fail(DG_ERR_ARG, "NULL argument");
    if (batch < 1 || canvas < 1 || canvas > 1024 || vocab < 1 || vocab > 524288)
        return fail(DG_ERR_SHAPE, "need batch >= 1, 1 <= canvas <= 1024, 1 <= vocab <= 524288");
    if (p->max_steps < 1 || step < 0) return fail(DG_ERR_ARG, "bad step / max_steps");
    if (p->top_k < 0 || p->top_k > dg::kTopKMax || p->top_k > vocab)
        return fail(DG_ERR_ARG, "top_k %d outside [0, min(64, vocab)]", p->top_k);
    if (p->lock_rule != DG_LOCK_MAXPROB && p->lock_rule != DG_LOCK_CUMENT)
        return fail(DG_ERR_ARG, "lock_rule %d", p->lock_rule);
    if (!(p->temp_start > 0.f) || !(p->temp_end > 0.f))
        return fail(DG_ERR_ARG, "temperatures must be positive");
    size_t need;
    dg_sampler_workspace_bytes(batch, canvas, &need);
    if (ws_bytes < need) return fail(DG_ERR_CAPACITY, "sampler workspace needs %zu bytes", need);
    // temperature of this step: linear from temp_start to temp_end over the budget
    double T = (double)p->temp_start;
    if (p->max_steps > 1)
        T = (double)p->temp_start + ((double)p->temp_end - (double)p->temp_start) * (double)step /
                                        (double)(p->max_steps - 1);
    const float Tf = (float)T;
    Carver cv(d_ws, ws_bytes);
    dg::SampleArgs a;
    a.B = batch;
    a.N = canvas;
    a.V = vocab;
    a.step = step;
    a.lock_rule = p->lock_rule;
    a.theta = p->lock_theta;
    a.tau = p->stop_tau;
    a.inv_t = 1.0f / Tf;
    a.require_stable = p->require_stable;
    a.max_steps = p->max_steps;
    a.seed = p->seed;
    a.logits = d_logits;
    a.canvas = d_canvas;
    a.argmax = d_argmax;
    a.lock = d_lock;
    a.stats = d_stats;
    a.stop = d_stop;
    a.y = cv.take<int32_t>((size_t)batch * canvas);
    a.r = cv.take<int32_t>((size_t)batch * canvas);
    a.newmax = cv.take<int32_t>((size_t)batch * canvas);
    a.nstop = nstop;
    a.halt = halt;
    a.host_stop = host_stop;
    a.trace = trace;
    if (probs) {
        // also write the next round's self-conditioning operand
        if (!rowmax || vocab % 128) return fail(DG_ERR_SHAPE, "probabilities need row maxima and vocab %% 128 == 0");
        a.rowmax = rowmax;
        a.rowmax_n = vocab / 64;
        a.probs = (uint16_t*)probs;
        a.probs_tiled = probs_tiled;
    }
    if (p->top_k > 0) {
        // top-k truncation; the block loop passes the head's slab maxima and
        // keeps the candidates for the next round's self-conditioning
        a.top_k = p->top_k;
        a.rowmax = rowmax;
        a.rowmax_n = rowmax ? cdiv(vocab, 64) : 0;
        a.probs = nullptr;
        a.tk_idx = tk_idx;
        a.tk_p = tk_p;
    }
    if (untimed) DG_HIP(dg::sample_update(a, st));
    else DG_HIP(timed(DG_TIMER_SAMPLER, st, [&] { return dg::sample_update(a, st); }));
    return DG_OK;
}

dg_status dg_sample_update_static(const dg_sampler_params* p, int32_t step, int32_t batch,
                                  int32_t canvas, int32_t vocab, const float* d_logits,
                                  int32_t* d_canvas, int32_t* d_argmax, uint8_t* d_lock,
                                  float* d_stats, int32_t* d_stop, void* stream) {
    if (batch < 1 || canvas < 1) return fail(DG_ERR_SHAPE, "need batch >= 1 and canvas >= 1");
    if ((long)batch * canvas > kStaticSamplerRows)
        return fail(DG_ERR_CAPACITY, "batch * canvas = %ld exceeds the static scratch's %d rows",
                    (long)batch * canvas, kStaticSamplerRows);
    void* ws = nullptr;
    DG_TRY(static_scratch(&ws));
    return sample_impl(p, step, batch, canvas, vocab, d_logits, d_canvas, d_argmax, d_lock,
                       d_stats, d_stop, ws, kStaticSamplerBytes, as_stream(stream), nullptr,
                       nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr, true);
}

dg_status dg_sample_update(const dg_sampler_params* p, int32_t step, int32_t batch,
                           int32_t canvas, int32_t vocab, const float* d_logits,
                           int32_t* d_canvas, int32_t* d_argmax, uint8_t* d_lock,
                           float* d_stats, int32_t* d_stop, void* d_ws, size_t ws_bytes,
                           void* stream) {
    return sample_impl(p, step, batch, canvas, vocab, d_logits, d_canvas, d_argmax, d_lock,
                       d_stats, d_stop, d_ws, ws_bytes, as_stream(stream));
}

dg_status dg_sample_update_probs(const dg_sampler_params* p, int32_t step, int32_t batch,
                                 int32_t canvas, int32_t vocab, const float* d_logits,
                                 int32_t* d_canvas, int32_t* d_argmax, uint8_t* d_lock,
                                 float* d_stats, int32_t* d_stop, const float* d_rowmax,
                                 int32_t blocked, void* d_probs, void* d_ws, size_t ws_bytes,
                                 void* stream) {
    if (!d_rowmax || !d_probs) return fail(DG_ERR_ARG, "NULL argument");
    return sample_impl(p, step, batch, canvas, vocab, d_logits, d_canvas, d_argmax, d_lock,
                       d_stats, d_stop, d_ws, ws_bytes, as_stream(stream), nullptr, nullptr,
                       d_rowmax, d_probs, blocked ? 1 : 0);
}

dg_status dg_stage_probs(int32_t T, int32_t vocab, int32_t blocked, const float* d_logits,
                         const float* d_stats, void* d_probs, void* stream) {
    if (!d_logits || !d_stats || !d_probs) return fail(DG_ERR_ARG, "NULL argument");
    if (T < 1 || vocab < 4 || vocab % 4) return fail(DG_ERR_SHAPE, "need T >= 1 and vocab %% 4 == 0");
    if (blocked && vocab % 64) return fail(DG_ERR_SHAPE, "the blocked layout needs vocab %% 64 == 0");
    DG_HIP(dg::selfcond_probs(d_logits, d_stats, (uint16_t*)d_probs, T, vocab, nullptr,
                                 blocked ? 1 : 0, as_stream(stream)));
    return DG_OK;
}

dg_status dg_canvas_init(uint64_t seed, int32_t block_index, int32_t batch, int32_t canvas,
                         int32_t vocab, int32_t* d_canvas, void* stream) {
    if (!d_canvas || batch < 1 || canvas < 1 || vocab < 1)
        return fail(DG_ERR_ARG, "bad canvas_init arguments");
    DG_HIP(dg::canvas_init(seed, block_index, batch, canvas, vocab, d_canvas, as_stream(stream)));
    return DG_OK;
}

// generate workspace: model scratch, then the loop's own buffers
static void carve_generate(Carver& cv, const dg_model* m, int B, Scratch& s, float** logits,
                           float** stats, int32_t** canvas, int32_t** argmax, uint8_t** lock,
                           int32_t** stop, void** sws, size_t* sws_bytes) {
    carve_scratch(cv, m, B, s);
    const size_t Tc = (size_t)B * m->c.canvas;
    logits[0] = cv.take<float>(Tc * m->c.vocab);
    logits[1] = cv.take<float>(Tc * m->c.vocab);
    stats[0] = cv.take<float>(Tc * 4);
    stats[1] = cv.take<float>(Tc * 4);
    *canvas = cv.take<int32_t>(Tc);
    *argmax = cv.take<int32_t>(Tc);
    *lock = cv.take<uint8_t>(Tc);
    *stop = cv.take<int32_t>(B + 2);   // flags, then count of stopped and the halt flag
    dg_sampler_workspace_bytes(B, m->c.canvas, sws_bytes);
    *sws = cv.take_bytes(*sws_bytes);
}

dg_status dg_generate_workspace_bytes(const dg_model* m, int32_t batch, size_t* bytes) {
    DG_TRY(check_model(m));
    if (!bytes || batch < 1) return fail(DG_ERR_ARG, "bad workspace request");
    Carver cv(nullptr, 0);
    Scratch s;
    float *lg[2], *stt[2];
    int32_t *cv_, *am, *sp;
    uint8_t* lk;
    void* sws;
    size_t sb;
    carve_generate(cv, m, batch, s, lg, stt, &cv_, &am, &lk, &sp, &sws, &sb);
    *bytes = cv.off + 256;
    return DG_OK;
}

// The block loop reads each round's stop flags from pinned host memory:
// two slots (one per round parity) of up to DG_MAX_LOOP_BATCH flags, allocated
// with the model so that no call of the loop allocates.
static dg_status check_loop_batch(const dg_model* m, int batch) {
    if (!m->hflags || !m->flag_ev[0] || !m->flag_ev[1])
        return fail(DG_ERR_HIP, "the model's stop-flag buffers were not allocated at creation");
    if (batch > m->hflags_cap)
        return fail(DG_ERR_CAPACITY, "block loop batch %d > %d", batch, m->hflags_cap);
    return DG_OK;
}

static dg_status generate_block_impl(dg_model* m, dg_kv* kv, int32_t batch,
                                     const dg_sampler_params* p, int32_t block_index,
                                     int32_t* d_block_out, int32_t* h_steps_out, float* d_trace,
                                     void* d_ws, size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!kv || !p || !d_block_out || !h_steps_out || !d_ws) return fail(DG_ERR_ARG, "NULL argument");
    if (batch != kv->B) return fail(DG_ERR_SHAPE, "batch %d != cache batch %d", batch, kv->B);
    const dg_config& c = m->c;
    if (kv->len + c.canvas > kv->cap)
        return fail(DG_ERR_CAPACITY, "cache needs len %d + canvas %d <= capacity %d", kv->len,
                    c.canvas, kv->cap);
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    float *lg[2], *stt[2];
    int32_t *canvas, *argmax, *stop;
    uint8_t* lock;
    void* sws;
    size_t sws_bytes;
    carve_generate(cv, m, batch, s, lg, stt, &canvas, &argmax, &lock, &stop, &sws, &sws_bytes);
    if (!cv.ok) return fail(DG_ERR_CAPACITY, "workspace of %zu bytes too small (need %zu)",
                            ws_bytes, cv.off);
    hipStream_t st = as_stream(stream);
    const size_t Tc = (size_t)batch * c.canvas;
    DG_TRY(check_loop_batch(m, batch));
    DG_HIP(dg::canvas_init(p->seed, block_index, batch, c.canvas, c.vocab, canvas, st));
    DG_HIP(dg::fill_i32(argmax, 0, (long)Tc, st));
    DG_HIP(dg::fill_i32(stop, 0, batch + 2, st));
    int32_t* nstop = stop + batch;
    int32_t* halt = stop + batch + 1;
    s.halt = halt;
    for (int b = 0; b < batch; ++b) h_steps_out[b] = 0;
    // The stop flags of round t (written by the canvas kernel straight into
    // pinned host memory, slot t & 1) are read on the host while round t+1
    // is already queued (one round of look-ahead hides the host round trip).
    // Once every sequence has stopped the sampler raises `halt` on the
    // device, so a look-ahead round after the last stop skips its heavy
    // kernels and leaves canvas, argmax and locks untouched.
    int nonfinite = -1;   // first canvas whose logits were not all finite
    int nonfinite_round = 0;
    auto flags_of = [&](int t, bool* all) -> dg_status {   // round t's flags; all stopped?
        DG_HIP(hipEventSynchronize(m->flag_ev[t & 1]));
        const int32_t* hs = m->hflags + (size_t)(t & 1) * m->hflags_cap;
        *all = true;
        for (int b = 0; b < batch; ++b) {
            if (h_steps_out[b] == 0 && hs[b]) {
                h_steps_out[b] = t + 1;
                if (hs[b] == 2 && nonfinite < 0) {
                    nonfinite = b;
                    nonfinite_round = t;
                }
            }
            *all = *all && hs[b];
        }
        return DG_OK;
    };
    // Blocked models: the sampler writes the self-conditioning probabilities
    // of round t while it reads round t's logits (the head GEMM supplies the
    // row maxima), so round t+1 skips the separate probability pass.  The
    // values are the same bits that pass would write.
    s.fuse = p->selfcond_on && p->top_k == 0 && m->blocked && m->embed_head;
    s.topk = p->selfcond_on ? p->top_k : 0;
    s.want_rowmax = (s.fuse || p->top_k > 0) && m->blocked && m->embed_head;
    const float* prev = nullptr;
    const float* prev_stats = nullptr;
    int t = 0;
    bool done = false;
    for (; t < p->max_steps && !done; ++t) {
        float* logits = lg[t & 1];
        float* stats = stt[t & 1];
        s.probs_ready = s.fuse && t > 0;
        s.topk_ready = s.topk > 0 && t > 0;
        if (c.dtype == DG_BF16)
            DG_TRY(denoise<bf16_t>(m, kv, batch, canvas, prev, prev_stats, logits, s, st));
        else
            DG_TRY(denoise<float>(m, kv, batch, canvas, prev, prev_stats, logits, s, st));
        DG_TRY(sample_impl(p, t, batch, c.canvas, c.vocab, logits, canvas, argmax, lock, stats,
                           stop, sws, sws_bytes, st, nstop, halt,
                           s.want_rowmax ? s.tmax : nullptr, s.fuse ? s.probs : nullptr,
                           s.probs_tiled, m->hflags + (size_t)(t & 1) * m->hflags_cap,
                           s.topk > 0 ? s.tk_idx : nullptr, s.topk > 0 ? s.tk_p : nullptr,
                           false, d_trace ? d_trace + (size_t)t * batch * 2 : nullptr));
        DG_HIP(hipEventRecord(m->flag_ev[t & 1], st));
        if (t > 0) DG_TRY(flags_of(t - 1, &done));
        if (p->selfcond_on) {
            prev = logits;
            prev_stats = stats;
        }
    }
    // the last round queued: its flags (a look-ahead round after the final
    // stop changes nothing)
    if (!done && t > 0) {
        bool all;
        DG_TRY(flags_of(t - 1, &all));
    }
    for (int b = 0; b < batch; ++b)
        if (h_steps_out[b] == 0) h_steps_out[b] = p->max_steps;
    DG_HIP(hipMemcpyAsync(d_block_out, argmax, Tc * sizeof(int32_t), hipMemcpyDeviceToDevice, st));
    if (nonfinite >= 0)
        return fail(DG_ERR_NONFINITE, "canvas %d: non-finite logits in round %d (block not committed)",
                    nonfinite, nonfinite_round);
    const size_t model_ws = ws_bytes;  // the model scratch is the prefix of d_ws
    return dg_commit_block(m, kv, batch, d_block_out, d_ws, model_ws, stream);
}

dg_status dg_generate_block(dg_model* m, dg_kv* kv, int32_t batch, const dg_sampler_params* p,
                            int32_t block_index, int32_t* d_block_out, int32_t* h_steps_out,
                            void* d_ws, size_t ws_bytes, void* stream) {
    return generate_block_impl(m, kv, batch, p, block_index, d_block_out, h_steps_out, nullptr,
                               d_ws, ws_bytes, stream);
}

dg_status dg_generate_block_trace(dg_model* m, dg_kv* kv, int32_t batch,
                                  const dg_sampler_params* p, int32_t block_index,
                                  int32_t* d_block_out, int32_t* h_steps_out, float* d_trace,
                                  void* d_ws, size_t ws_bytes, void* stream) {
    if (!d_trace) return fail(DG_ERR_ARG, "NULL trace");
    return generate_block_impl(m, kv, batch, p, block_index, d_block_out, h_steps_out, d_trace,
                               d_ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ stages
dg_status dg_stage_input(dg_model* m, int32_t batch, const int32_t* d_canvas,
                         const float* d_prev_logits, const float* d_prev_stats, float* d_h,
                         void* d_ws, size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!d_canvas || !d_h || batch < 1) return fail(DG_ERR_ARG, "bad arguments");
    if ((d_prev_logits == nullptr) != (d_prev_stats == nullptr))
        return fail(DG_ERR_ARG, "prev_logits and prev_stats must both be set or both NULL");
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, batch, d_ws, ws_bytes, s, cv));
    if (m->c.dtype == DG_BF16)
        return stage_input<bf16_t>(m, batch, d_canvas, d_prev_logits, d_prev_stats, d_h, s,
                                       as_stream(stream));
    return stage_input<float>(m, batch, d_canvas, d_prev_logits, d_prev_stats, d_h, s,
                              as_stream(stream));
}

dg_status dg_stage_input_topk(dg_model* m, int32_t batch, const int32_t* d_canvas,
                              const float* d_prev_logits, int32_t top_k, float* d_h, void* d_ws,
                              size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!d_canvas || !d_h || !d_prev_logits || batch < 1) return fail(DG_ERR_ARG, "bad arguments");
    if (top_k < 1 || top_k > dg::kTopKMax || top_k > m->c.vocab)
        return fail(DG_ERR_ARG, "top_k %d outside [1, min(64, vocab)]", top_k);
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, batch, d_ws, ws_bytes, s, cv));
    s.topk = top_k;
    if (m->c.dtype == DG_BF16)
        return stage_input<bf16_t>(m, batch, d_canvas, d_prev_logits, nullptr, d_h, s,
                                   as_stream(stream));
    return stage_input<float>(m, batch, d_canvas, d_prev_logits, nullptr, d_h, s,
                              as_stream(stream));
}

dg_status dg_stage_attention(dg_model* m, dg_kv* kv, int32_t layer, int32_t batch, int32_t n,
                             int32_t causal, float* d_h, void* d_ws, size_t ws_bytes,
                             void* stream) {
    DG_TRY(check_model(m));
    if (!kv || !d_h || layer < 0 || layer >= m->c.n_layers || n < 1)
        return fail(DG_ERR_ARG, "bad arguments");
    if (batch != kv->B) return fail(DG_ERR_SHAPE, "batch %d != cache batch %d", batch, kv->B);
    if (kv->len + n > kv->cap) return fail(DG_ERR_CAPACITY, "len + n exceeds capacity");
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, batch, d_ws, ws_bytes, s, cv));
    if (batch * n > token_budget(m, batch))
        return fail(DG_ERR_CAPACITY, "batch*n exceeds the workspace token budget");
    if (m->c.dtype == DG_BF16)
        return attn_half<bf16_t>(m, kv, layer, batch, n, kv->len, causal != 0, d_h, s,
                                     as_stream(stream));
    return attn_half<float>(m, kv, layer, batch, n, kv->len, causal != 0, d_h, s,
                            as_stream(stream));
}

dg_status dg_stage_moe(dg_model* m, int32_t layer, int32_t T, float* d_h, int32_t* d_route,
                       float* d_gates, void* d_ws, size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!d_h || layer < 0 || layer >= m->c.n_layers || T < 1) return fail(DG_ERR_ARG, "bad arguments");
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, 1, d_ws, ws_bytes, s, cv));
    if (T > token_budget(m, 1)) return fail(DG_ERR_CAPACITY, "T exceeds the workspace token budget");
    hipStream_t st = as_stream(stream);
    if (m->c.dtype == DG_BF16) DG_TRY(moe_half<bf16_t>(m, layer, T, d_h, s, st));
    else DG_TRY(moe_half<float>(m, layer, T, d_h, s, st));
    if (d_route)
        DG_HIP(hipMemcpyAsync(d_route, s.route, (size_t)T * m->c.top_k * sizeof(int32_t),
                              hipMemcpyDeviceToDevice, st));
    if (d_gates)
        DG_HIP(hipMemcpyAsync(d_gates, s.gates, (size_t)T * m->c.top_k * sizeof(float),
                              hipMemcpyDeviceToDevice, st));
    return DG_OK;
}

dg_status dg_stage_head_rowmax(dg_model* m, int32_t T, const float* d_h, float* d_logits,
                               float* d_rowmax, void* d_ws, size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!d_h || !d_logits || !d_rowmax || T < 1) return fail(DG_ERR_ARG, "bad arguments");
    if (!m->blocked || !m->embed_head)
        return fail(DG_ERR_UNSUPPORTED, "row maxima come from the blocked head (embed_head)");
    const int nb = std::max(1, cdiv(T, m->c.canvas));
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, nb, d_ws, ws_bytes, s, cv));
    if (T > token_budget(m, nb)) return fail(DG_ERR_CAPACITY, "T exceeds the workspace token budget");
    if (T > s.ut_rows) return fail(DG_ERR_CAPACITY, "T exceeds the head's blocked row budget %d", s.ut_rows);
    s.want_rowmax = true;
    s.tmax = d_rowmax;
    return stage_head<bf16_t>(m, T, d_h, d_logits, s, as_stream(stream));
}

dg_status dg_stage_head(dg_model* m, int32_t T, const float* d_h, float* d_logits, void* d_ws,
                        size_t ws_bytes, void* stream) {
    DG_TRY(check_model(m));
    if (!d_h || !d_logits || T < 1) return fail(DG_ERR_ARG, "bad arguments");
    const int nb = std::max(1, cdiv(T, m->c.canvas));
    Carver cv(d_ws, ws_bytes);
    Scratch s;
    DG_TRY(check_ws(m, nb, d_ws, ws_bytes, s, cv));
    if (T > token_budget(m, nb)) return fail(DG_ERR_CAPACITY, "T exceeds the workspace token budget");
    if (m->c.dtype == DG_BF16)
        return stage_head<bf16_t>(m, T, d_h, d_logits, s, as_stream(stream));
    return stage_head<float>(m, T, d_h, d_logits, s, as_stream(stream));
}

dg_status dg_timer_enable(uint32_t mask) {
    g_timers.clear();
    g_timers.mask = mask & ((1u << DG_TIMER_COUNT) - 1);
    return DG_OK;
}

dg_status dg_timer_read(int32_t id, double* total_ms, int64_t* launches) {
    if (id < 0 || id >= DG_TIMER_COUNT || !total_ms || !launches)
        return fail(DG_ERR_ARG, "bad timer read");
    double tot = 0.0;
    for (auto& p : g_timers.ev[id]) {
        DG_HIP(hipEventSynchronize(p.second));
        float ms = 0.f;
        DG_HIP(hipEventElapsedTime(&ms, p.first, p.second));
        tot += ms;
    }
    *total_ms = tot;
    *launches = (int64_t)g_timers.ev[id].size();
    return DG_OK;
}

}  // extern "C"
