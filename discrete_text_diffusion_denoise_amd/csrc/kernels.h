// Host-side launchers of the gfx950 kernels (internal to libdg.so).
// Every launcher enqueues on `st` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// ------------------------------------------------------------------ GEMM
enum { EPI_STORE_F32 = 0, EPI_ADD_F32 = 1, EPI_SPLITK = 2, EPI_EMBED_ADD = 3 };

struct GemmArgs {
    int M = 0, N = 0, K = 0;
    const void* A = nullptr;        // [M][lda] of T (amode 0) or fp32 logits (amode 1)
    long lda = 0;
    const int32_t* a_rows = nullptr;  // optional row gather for A (amode 0)
    const float* a_stats = nullptr;   // amode 1: per-row {max, sum, ...}, stride 4
    const void* B = nullptr;        // [N][ldb] of T
    long ldb = 0;
    void* C = nullptr;              // fp32 [M][ldc] (split-K: [splits][M][ldc])
    long ldc = 0;
    int k_split = 0;                // K elements per split (multiple of 64)
    const void* E = nullptr;        // EPI_EMBED_ADD: embedding [vocab][lde] of T
    long lde = 0;
    int vocab = 0;
    const int32_t* tokens = nullptr;  // EPI_EMBED_ADD: token per row
    int E_is_f32 = 0;               // split-K epilogue: E element type
    int xcd_group = 0;              // put a k-split's column tiles on one XCD
    int k_rotate = 0;               // rotate each tile's starting k-slice
    const int32_t* halt = nullptr;  // vocabulary GEMMs: skip all work when *halt != 0
    int b_bf16 = 0;                 // fp32 GEMM: B is bf16, widened on load
    // column segments: columns [n_b2, n_b3) are rows of B2, [n_b3, N) rows
    // of B3 (0 = no segment); the stacked Q/K/V projection in one product
    const void* B2 = nullptr;
    const void* B3 = nullptr;
    int n_b2 = 0, n_b3 = 0;
    // bf16 ring kernel: operand stored in 256 x 32 blocks (1, see
    // tiled_index) or, for A, 256 x 64 blocks (2, tiled64_index); lda / ldb
    // are then ignored and the row count is padded to 256
    int a_tiled = 0, b_tiled = 0;
    // bf16 ring kernel, EPI_STORE_F32 with N % 64 == 0: per-row maxima of
    // each 64-column slab, rowmax[m * (N / 64) + n / 64] (the row maxima of
    // the logits, before they are read again)
    float* rowmax = nullptr;
};

// Blocked layout of a bf16 matrix [R][K] (K a multiple of 32, R padded to a
// multiple of 256): rows in tiles of 256, each tile's K in stages of 32, one
// stage of one tile = 256 rows x 32 values = 16 KiB, contiguous.  Element
// (r, k) sits at ((r / 256 * (K / 32) + k / 32) * 256 + r % 256) * 32 + k % 32.
__host__ __device__ __forceinline__ long tiled_index(long r, long k, long K) {
    return (((r >> 8) * (K >> 5) + (k >> 5)) * 256 + (r & 255)) * 32 + (k & 31);
}

// The same with 64-value stages (256 rows x 64 values = 32 KiB, contiguous;
// K a multiple of 64): one row's stage is a whole 128-byte line, which the
// sampler's row pass writes at once.
__host__ __device__ __forceinline__ long tiled64_index(long r, long k, long K) {
    return (((r >> 8) * (K >> 6) + (k >> 6)) * 256 + (r & 255)) * 64 + (k & 63);
}

// Row n of the (segmented) B operand, in elements of type E.
template <typename E>
__device__ __forceinline__ const E* b_row(const GemmArgs& g, int n) {
    if (g.n_b3 && n >= g.n_b3) return reinterpret_cast<const E*>(g.B3) + (long)(n - g.n_b3) * g.ldb;
    if (g.n_b2 && n >= g.n_b2) return reinterpret_cast<const E*>(g.B2) + (long)(n - g.n_b2) * g.ldb;
    return reinterpret_cast<const E*>(g.B) + (long)n * g.ldb;
}

// C (op)= A * B^T.  amode 1 reads A as softmax of fp32 logits (only with
// EPI_SPLITK).  T = bf16_t (uint16_t) or float.
template <typename T>
hipError_t gemm_tn(const GemmArgs& g, int amode, int epi, int splits, hipStream_t st);

// bf16 C (STORE_F32 or SPLITK) = A * B^T with direct-to-LDS loads and a
// four-stage ring (256 x 256 tiles).  gemm_dma_ok says whether the operands
// meet its conditions: K and k_split multiples of 128, 16-byte aligned rows,
// no row gather.
// Decode-step head: M <= 16 rows (A and B blocked, K <= 2048, N % 256 == 0),
// EPI_STORE_F32, optional 64-column slab maxima (rowmax)
bool gemm_decode_ok(const GemmArgs& g);
hipError_t gemm_decode(const GemmArgs& g, hipStream_t st);
bool gemm_dma_ok(const GemmArgs& g, int epi);
hipError_t gemm_dma_bf16(const GemmArgs& g, int epi, int splits, hipStream_t st);
// Skinny ring kernel (256 x 64 tiles, row-major bf16 operands, segmented B
// allowed): writes split-K partials C[kz][M][ldc]; K and k_split multiples
// of 128.
bool gemm_skinny_ok(const GemmArgs& g);
hipError_t gemm_skinny_splitk(const GemmArgs& g, int splits, hipStream_t st);

// Streaming bf16 GEMM (M <= 256 per row tile): all rows of a tile share the A
// slice in LDS, each wave streams 16*tn columns of B (tn = 1 or 4).
hipError_t gemm_stream(const GemmArgs& g, int epi, int tn, int splits, hipStream_t st);
int stream_tm_for(int M);
// C[m][n] (epi)= sum_z part[z][m][n]  (part is [splits][M][N])
hipError_t splitk_epilogue(const GemmArgs& g, const float* part, int splits, int epi,
                           hipStream_t st);

// ------------------------------------------------------------------ elementwise
hipError_t fill_i32(int32_t* p, int32_t v, long n, hipStream_t st);
// RMSNorm into the blocked bf16 layout (tiled_index over [rows][d])
hipError_t rmsnorm_tiled(const float* h, const float* w, uint16_t* u, int rows, int d, float eps,
                         hipStream_t st);
// E [V][d] (bf16) into the blocked layout of E (transpose 0: rows V padded to
// 256, K = d) or of E^T (transpose 1: rows d, K = V; d % 256 == 0, V % 32 == 0)
hipError_t embed_tile(const uint16_t* E, int V, int d, int transpose, uint16_t* out,
                      hipStream_t st);
// u[t] = h[t] / sqrt(mean(h[t]^2) + eps) * w   (u in T; also fp32 into u32 if
// set, and MXFP8 codes / scale codes into q8 [rows][d] / q8s [rows][d/32] if set)
template <typename T>
hipError_t rmsnorm(const float* h, const float* w, T* u, int rows, int d, float eps,
                   hipStream_t st, float* u32 = nullptr, uint8_t* q8 = nullptr,
                   uint8_t* q8s = nullptr);
// h[b*n + i] = E[tok[b*ld + i]] (fp32), b < B, i < n; E has V rows
template <typename T>
hipError_t embed_rows(const T* E, int V, const int32_t* tok, int ld, int n, int B, float* h, int d,
                      hipStream_t st);
// out[t][j] = sum_s part[s][t][j]  (T); with row_stats, times 1 / row_stats[t][1]
template <typename T>
hipError_t splitk_reduce(const float* part, T* out, int splits, int rows, int cols,
                         hipStream_t st, const float* row_stats = nullptr);
// out[i] = float(in[i])
hipError_t widen_bf16(const uint16_t* in, float* out, long n, hipStream_t st);
// out[j][v] = E[v][j]
template <typename T>
hipError_t transpose(const T* in, T* out, int rows, int cols, hipStream_t st);

// RoPE on q and k (fp32 qkv [B*n][(Hq+2Hkv)*dh]); q -> q_out [B*n][Hq*dh] (T);
// k, v -> cache slots [pos0, pos0+n) of kc/vc [B][Hkv][cap][dh] (T, one layer).
template <typename T>
hipError_t rope_kv(const float* qkv, T* q_out, T* kc, T* vc, int B, int n, int pos0, int cap,
                   int Hq, int Hkv, int dh, int rope_on, float theta, hipStream_t st);
// rope_kv from the stacked Q/K/V product's split-K partials [splits][B*n][width]
// (summed as splitk_epilogue sums them)
template <typename T>
hipError_t splitk_rope_kv(const float* part, int splits, T* q_out, T* kc, T* vc, int B, int n,
                          int pos0, int cap, int Hq, int Hkv, int dh, int rope_on, float theta,
                          hipStream_t st);
// h [rows][d] += the split-K partials part [splits][rows][d] (summed as
// splitk_epilogue sums them), then rmsnorm of the new rows with its outputs
template <typename T>
hipError_t splitk_add_norm(const float* part, int splits, float* h, int rows, int d,
                           const float* w, T* u, float eps, hipStream_t st, float* u32,
                           uint8_t* q8, uint8_t* q8s);

// ------------------------------------------------------------------ attention
struct AttnArgs {
    const void* q = nullptr;   // [B*n][Hq*dh] (T)
    const void* kc = nullptr;  // [B][Hkv][cap][dh] (T)
    const void* vc = nullptr;
    void* out = nullptr;       // [B*n][Hq*dh] (T)
    float* part_o = nullptr;   // [splits][B*n][Hq][dh]   (splits > 1)
    float* part_ml = nullptr;  // [splits][B*n][Hq][2]
    int B = 0, n = 0, pos0 = 0, cap = 0, Hq = 0, Hkv = 0, dh = 0;
    int kv_len = 0;            // keys [0, kv_len)
    int causal = 0;            // query i (position pos0+i) sees keys <= pos0+i
    int splits = 1;
    int split_len = 0;         // keys per split (multiple of 32)
    const int32_t* halt = nullptr;   // skip all work when *halt != 0
};
template <typename T>
hipError_t attention(const AttnArgs& a, hipStream_t st);
// Number of key splits the launcher would use for this shape.
int attention_splits(int B, int n, int Hq, int Hkv, int kv_len, int causal, int max_splits,
                     int* split_len, int dh, bool bf16);

// ------------------------------------------------------------------ MoE
struct MoeArgs {
    int T = 0, d = 0, E = 0, k = 0, F = 0;
    const float* z = nullptr;        // router logits [T][E]
    int32_t* route = nullptr;        // [T][k] experts, selection order
    float* gates = nullptr;          // [T][k]
    int32_t* counts = nullptr;       // [E]
    int32_t* offsets = nullptr;      // [E+1]
    int32_t* order = nullptr;        // optional [E]: experts by falling count (ties: lower id)
    int32_t* perm_tok = nullptr;     // [T*k] token of each sorted slot
    int32_t* slot_of = nullptr;      // [T*k] sorted slot of (t, j)
    const void* u = nullptr;         // normalised tokens [T][d] (T)
    const void* w_gate = nullptr;    // [E][F][d]
    const void* w_up = nullptr;      // [E][F][d]
    const void* w_down = nullptr;    // [E][d][F]
    void* act = nullptr;             // [T*k][F] (T)
    float* y = nullptr;              // [T*k][d]
    float* h = nullptr;              // residual [T][d]
    int k_rotate = 0;                // rotate each block's starting k-stage
    const int32_t* halt = nullptr;   // expert kernels: skip all work when *halt != 0
    // 8-bit experts: w_gate / w_up / w_down hold E4M3 codes in the tiled
    // layout of quantize_fp8, one fp32 scale per weight row (s_gate, s_up
    // [E][F]; s_down [E][d])
    int f8 = 0;
    const float* s_gate = nullptr;
    const float* s_up = nullptr;
    const float* s_down = nullptr;
    // MXFP4 experts: w_gate / w_up / w_down hold packed E2M1 codes and x_*
    // the E8M0 scale codes of each 32-k block, both in the tiled layout of
    // quantize_mxfp4 (rows E*R, columns K)
    int f4 = 0;
    const uint8_t* x_gate = nullptr;
    const uint8_t* x_up = nullptr;
    const uint8_t* x_down = nullptr;
    // quantised experts take MXFP8 activations (E4M3 codes, an E8M0 scale
    // code per 32 features): the normalised tokens u8 [T][d] / u8s [T][d/32]
    // (written by the RMSNorm) and the gate/up output act8 [T*k][F] / act8s
    // [T*k][F/32] (written by the gate/up epilogue)
    const uint8_t* u8 = nullptr;
    const uint8_t* u8s = nullptr;
    uint8_t* act8 = nullptr;
    uint8_t* act8s = nullptr;
    // optional [E+1]: exclusive prefix, over the experts in `order`, of their
    // chunks of kMoeChunk tokens (written with `order` by moe_route): the
    // work items (expert, chunk) of the block-scaled expert kernels
    int32_t* work = nullptr;
    // optional [cdiv(T*k, kMoeChunk) + E][4] (16-byte aligned): per work
    // item, written with `work` once the offsets are known, (its expert, the
    // expert's first routed row, the item's first row within the expert, the
    // expert's row count), so a block finds its item with one load
    int32_t* items = nullptr;
    // optional: router logits computed inside the routing (moe_route) from
    // the fp32 normalised tokens router_u [T][d] and the bf16 router rows
    // router_w [E][d], instead of reading z; used where router_fused_ok
    const float* router_u = nullptr;
    const void* router_w = nullptr;
};
constexpr int kMoeChunk = 64;
// shapes the fused router + top-k kernel takes: few tokens (one workgroup
// each), d of 512, 1024 or 2048, at most 256 experts
inline bool router_fused_ok(int T, int d, int E) {
    return T >= 1 && T <= 512 && (d == 512 || d == 1024 || d == 2048) && E >= 1 && E <= 256;
}
// compute units of the current device (cached per device)
int cu_count();
// routing, counts and the stable permutation
hipError_t moe_route(const MoeArgs& a, hipStream_t st);
template <typename T>
hipError_t moe_gateup(const MoeArgs& a, hipStream_t st);
template <typename T>
hipError_t moe_down(const MoeArgs& a, hipStream_t st);
hipError_t moe_combine(const MoeArgs& a, hipStream_t st);
// moe_combine that also writes u = RMSNorm(new h rows, weight nw) (T), with
// the bits of moe_combine followed by rmsnorm; for k in {2, 4, 8}
bool moe_combine_norm_ok(int k);
template <typename T>
hipError_t moe_combine_norm(const MoeArgs& a, const float* nw, T* u, float eps, hipStream_t st);
// the bf16 ring kernels' shape limits (d and F multiples of 256)
bool expert_dma_ok(const MoeArgs& a);
// quantised experts (f4 or f8) on the block-scaled MFMA: d and F multiples of
// 128, MXFP8 activations in u8 / u8s, act8 / act8s written by the gate/up
// product and read by the down product
bool expert_mx_ok(const MoeArgs& a);
hipError_t moe_gateup_mx(const MoeArgs& a, hipStream_t st);
hipError_t moe_down_mx(const MoeArgs& a, hipStream_t st);

// E4M3 codes and per-row scales of src [rows][cols] (T = float or bf16_t;
// rows % 16 == 0, cols % 128 == 0): scale = max|x| / 448 (1 for a zero row),
// code = round-to-nearest-even of x / scale, saturating at 448.  Codes in the
// expert kernels' tiled layout: per 16-row tile and 128-column step, two
// 1-KiB halves (columns 0..63, 64..127), chunk 16 g + r of half h holding
// row r's columns 64 h + 16 g .. +15; the tile's steps follow one another
template <typename T>
hipError_t quantize_fp8(const T* src, long rows, int cols, uint8_t* q, float* scale,
                        hipStream_t st);

// MXFP4 codes and scale codes of src [rows][cols] (rows % 16 == 0, cols % 128
// == 0), in the expert kernels' tiled layout: per 16-row tile and 128-column
// step, 1 KiB of codes (chunk 16 g + r: row r's 32-column block g, two codes
// a byte, the even column low) and 64 scale codes (byte 16 g + r); the tile's
// steps follow one another, then the next tile
template <typename T>
hipError_t quantize_mxfp4(const T* src, long rows, int cols, uint8_t* q, uint8_t* scale,
                          hipStream_t st);

// ------------------------------------------------------------------ sampler
struct SampleArgs {
    int B = 0, N = 0, V = 0, step = 0;
    int lock_rule = 1;
    float theta = 0.1f, tau = 0.005f, inv_t = 1.0f;
    int require_stable = 1, max_steps = 48;
    uint64_t seed = 0;
    const float* logits = nullptr;   // [B][N][V]
    int32_t* canvas = nullptr;
    int32_t* argmax = nullptr;
    uint8_t* lock = nullptr;
    float* stats = nullptr;          // [B][N][4]
    int32_t* stop = nullptr;         // [B]
    int32_t* y = nullptr;            // scratch [B][N] drawn tokens
    int32_t* r = nullptr;            // scratch [B][N] renoise tokens
    int32_t* newmax = nullptr;       // scratch [B][N] argmax of this step
    int32_t* nstop = nullptr;        // optional: count of stopped sequences
    int32_t* halt = nullptr;         // optional: set to 1 once all B have stopped
    int32_t* host_stop = nullptr;    // optional: the stop flags also go here (pinned host memory)
    // optional [B][2]: a running canvas's mean entropy (the value the stop
    // rule tests) and its count of locked positions after this step; NaN and
    // 0 for a canvas reported non-finite; stopped canvases are not written
    float* trace = nullptr;
    // optional (V % 128 == 0): also write the self-conditioning weights of
    // the logits (selfcond_probs) as bf16 [B*N][V], 64-wide blocked
    // (probs_tiled, tiled64_index) or row-major, the operand of the next
    // round; the row maximum is taken from rowmax [B*N][rowmax_n] (the head
    // GEMM's slab maxima)
    const float* rowmax = nullptr;
    int rowmax_n = 0;
    uint16_t* probs = nullptr;
    int probs_tiled = 1;
    // top-k truncation (1 <= top_k <= 64; 0 = the full distribution): the
    // statistics, draw and argmax come from each row's top_k logits; the
    // slab maxima are read from rowmax when set (rowmax_n = V / 64), else
    // computed from the row.  tk_idx / tk_p (optional, [B*N][top_k]) receive
    // the candidates and their self-conditioning weights; list_only skips
    // everything else (the self-conditioning of a stand-alone step).
    int top_k = 0;
    int32_t* tk_idx = nullptr;
    float* tk_p = nullptr;
    int list_only = 0;
    // statistics only (the full distribution at T = 1): per row the
    // optional stats and newmax, and, when loss is set, the cross-entropy at
    // target[row]: L(S) - (l[target] - m), NaN for a target outside [0, V);
    // no draw, no canvas update, stop may be null
    int stats_only = 0;
    const int32_t* target = nullptr;
    float* loss = nullptr;
};
constexpr int kTopKMax = 64;
hipError_t sample_update(const SampleArgs& a, hipStream_t st);
// s[t][:] = sum_i p[t][i] * E[idx[t][i]][:] over i < K in order (fp32), stored
// in T; E [V][d] of T
template <typename T>
hipError_t selfcond_topk(const T* E, int d, const int32_t* idx, const float* p, int K, int rows,
                         T* out, hipStream_t st);
// Self-conditioning weights of logit rows [rows][V] with their statistics
// (stats[r][0] = row max): bf16, row-major or 64-wide blocked (`tiled`,
// tiled64_index, V % 64 == 0),
// the same bits the row pass writes through SampleArgs::probs; the division
// by stats[r][1] follows the product (splitk_reduce with row_stats).
// V % 4 == 0.  halt: when non-null and *halt != 0 the kernel does nothing.
hipError_t selfcond_probs(const float* logits, const float* stats, uint16_t* out, int rows, int V,
                          const int32_t* halt, int tiled, hipStream_t st);
hipError_t canvas_init(uint64_t seed, int block, int B, int N, int V, int32_t* canvas,
                       hipStream_t st);
// Multinomial corruption of the training-side forward: position (b, i)
// draws Philox counter (step, b, i, 2), key (seed, 0); it takes
// uniform_token(word 1, V) when uniform(word 0) < rate[b], else clean[b][i].
hipError_t corrupt(uint64_t seed, int step, int B, int N, int V, const float* rate,
                   const int32_t* clean, int32_t* out, hipStream_t st);
// mean = (sequential binary32 sum of loss[0 .. rows)) / rows, one thread
hipError_t mean_seq(const float* loss, int rows, float* mean, hipStream_t st);
// Greedy decoding: out[r * out_stride] = the index of row r's largest value,
// ties to the lower index (NaNs never win; an all-NaN row gives 0).
// logits [rows][V], 16-byte aligned.
hipError_t argmax_rows(const float* logits, int rows, int V, int32_t* out, long out_stride,
                       hipStream_t st);
// The same from the head's 64-column slab maxima rowmax [rows][V / 64]
// (V % 64 == 0), reading one slab of the logits per row.
hipError_t argmax_slabs(const float* logits, const float* rowmax, int rows, int V, int32_t* out,
                        long out_stride, hipStream_t st);

}  // namespace dg
