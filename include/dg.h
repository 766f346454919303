/*
 * dg.h -- C ABI of an MI355X-native denoising step for a block text-diffusion
 * mixture-of-experts language model.
 *
 * The method (pages on DiffusionGemma; citations name the page and section):
 *   - report-summary page (animattoys.com), section 1: a block of 256 tokens
 *     starts as uniformly random vocabulary tokens and is refined in
 *     parallel over rounds; uncertain positions are replaced by any
 *     vocabulary token (multinomial diffusion);
 *   - same page, section 2: one set of weights runs causal attention over
 *     the prompt and bidirectional attention over the canvas; 128 experts,
 *     8 active per token; a self-conditioning input from the previous round;
 *   - same page, section 4: entropy-ordered locking within a 0.1 entropy
 *     budget, re-randomisation of the rest, temperature 0.8 -> 0.4, stop on
 *     mean entropy < 0.005 with an unchanged most likely sequence, <= 48
 *     rounds;
 *   - youleyou.com article, "Architecture basis": the causal encoder fills a
 *     KV cache that every canvas position attends to; finished blocks are
 *     handed to the KV cache and the next canvas is conditioned on them
 *     (also akiraxclaw.com blog, "memory, not compute").
 *
 * Conventions for every call:
 *   - Device pointers ("d_" prefix) point to GPU memory owned by the caller;
 *     host pointers ("h_" prefix, or structs passed by pointer) are read
 *     during the call only.  The library never allocates device memory: all
 *     scratch space comes from a caller-supplied workspace.
 *   - Work is enqueued asynchronously on the given stream (a hipStream_t
 *     passed as void*; NULL = the default stream).  Only dg_generate_block
 *     waits on the stream (to read stop flags).
 *   - Every function returns a dg_status; on failure nothing has been
 *     enqueued (argument errors) or the HIP error is reported as DG_ERR_HIP.
 *     dg_last_error() gives a human-readable detail for the calling thread.
 *   - Token ids are int32 in [0, vocab).  Canvas length N is 256 in the
 *     pages' method; the library accepts any N in [1, 1024].
 *   - Weight layout: every linear map is [out_features][in_features],
 *     row-major, applied as y = x W^T, in the model dtype (fp32 or bf16).
 *     RMSNorm scales are fp32.  Weights are borrowed: they must stay valid
 *     while the model handle lives.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DG_OK = 0,
    DG_ERR_ARG = 1,         /* NULL pointer or out-of-range argument            */
    DG_ERR_SHAPE = 2,       /* shapes inconsistent or outside supported limits  */
    DG_ERR_DTYPE = 3,       /* unknown dtype                                    */
    DG_ERR_CAPACITY = 4,    /* KV cache or workspace too small                  */
    DG_ERR_NONFINITE = 5,   /* non-finite logits (dg_generate_block)            */
    DG_ERR_HIP = 6,         /* a HIP runtime call failed                        */
    DG_ERR_UNSUPPORTED = 7  /* valid request the library does not implement     */
} dg_status;

typedef enum {
    DG_F32 = 0,
    DG_BF16 = 1,
    DG_FP8_E4M3 = 2,  /* OCP 8-bit float E4M3 ("e4m3fn"), expert weights only */
    DG_MXFP4 = 3      /* OCP MXFP4: E2M1 codes with an E8M0 scale per 32,       */
                      /* expert weights only                                     */
} dg_dtype;

typedef enum {
    DG_LOCK_MAXPROB = 0,    /* lock i  <=>  max-probability(i) > theta                      */
    DG_LOCK_CUMENT = 1      /* entropy order, lock while running entropy <= theta (pages) */
} dg_lock_rule;

typedef struct {
    int32_t n_layers;
    int32_t d_model;
    int32_t n_heads;        /* query heads                                    */
    int32_t n_kv_heads;     /* key/value heads (n_heads % n_kv_heads == 0)    */
    int32_t head_dim;       /* even, <= 256, multiple of 32                   */
    int32_t n_experts;      /* <= 256                                         */
    int32_t top_k;          /* <= min(n_experts, 16)                          */
    int32_t d_ff;           /* expert hidden width (multiple of 32)           */
    int32_t vocab;          /* <= 524288                                      */
    int32_t canvas;         /* N, tokens per canvas                           */
    int32_t dtype;          /* dg_dtype of weights, KV cache, matmul operands */
    int32_t rope_on;        /* 1: rotate-half RoPE on q and k                 */
    float rope_theta;       /* RoPE base                                      */
    float rms_eps;          /* RMSNorm epsilon                                */
    int32_t expert_dtype;   /* 0: experts in `dtype`; DG_FP8_E4M3: expert     */
                            /* weights as E4M3 codes with per-row fp32 scales; */
                            /* DG_MXFP4: packed E2M1 codes with block scales   */
                            /* (both: bf16 models, d_model and d_ff multiples  */
                            /* of 256)                                         */
} dg_config;

typedef struct {
    const float* attn_norm;  /* [d]                 */
    const void* wq;          /* [Hq*dh][d]          */
    const void* wk;          /* [Hkv*dh][d]         */
    const void* wv;          /* [Hkv*dh][d]         */
    const void* wo;          /* [d][Hq*dh]          */
    const float* moe_norm;   /* [d]                 */
    const void* w_router;    /* [E][d]              */
    const void* w_gate;      /* [E][F][d]           */
    const void* w_up;        /* [E][F][d]           */
    const void* w_down;      /* [E][d][F]           */
    /* FP8 experts only (else NULL): w_gate / w_up / w_down hold E4M3 codes   */
    /* in the tiled layout of dg_quantize_fp8 (rows E*R, columns K), and these */
    /* one fp32 scale per weight row: weight[e][r][k] = decode(code) * s[e][r] */
    const float* s_gate;     /* [E][F]              */
    const float* s_up;       /* [E][F]              */
    const float* s_down;     /* [E][d]              */
    /* MXFP4 experts only (else NULL): w_gate / w_up / w_down hold E2M1 codes  */
    /* and these the E8M0 scale code of every 32-k block, both in the tiled    */
    /* layout of dg_quantize_mxfp4 (rows E*R, columns K), so that               */
    /* weight[e][r][k] = decode(code) * 2^(scale - 127)                        */
    const uint8_t* x_gate;   /* E*F*d/32 bytes      */
    const uint8_t* x_up;     /* E*F*d/32 bytes      */
    const uint8_t* x_down;   /* E*d*F/32 bytes      */
} dg_layer_weights;

typedef struct {
    const void* embed;       /* [V][d] tied embedding / output head                    */
    const void* embed_t;     /* E^T for self-conditioning, written by dg_embed_transpose */
                             /* (layout below); required for it, else may be NULL      */
    const void* w_sc;        /* [d][d] self-conditioning projection                    */
    const float* final_norm; /* [d]                                                    */
    const dg_layer_weights* layers; /* host array [n_layers], copied at create        */
    const void* embed_head;  /* optional: E in the blocked layout (dg_embed_head); NULL */
                             /* = the head reads `embed`                              */
} dg_weights;

typedef struct {
    int32_t lock_rule;       /* dg_lock_rule                                   */
    float lock_theta;        /* entropy budget (CUMENT) or probability (MAXPROB) */
    float temp_start;        /* temperature at step 0                          */
    float temp_end;          /* temperature at step max_steps-1 (linear)       */
    float stop_tau;          /* mean-entropy stop threshold (nats)             */
    int32_t require_stable;  /* 1: also require argmax unchanged from previous step */
    int32_t max_steps;       /* round budget (>= 1)                            */
    uint64_t seed;           /* Philox key                                     */
    int32_t selfcond_on;     /* dg_generate_block: feed previous logits back   */
    int32_t top_k;           /* 0: the full distribution; 1..64: top-k         */
                             /* truncation (report-summary page, section 9):  */
                             /* statistics, draw and self-conditioning use     */
                             /* each position's top_k logits only              */
} dg_sampler_params;

typedef struct dg_model dg_model;
typedef struct dg_kv dg_kv;

/* ---------------------------------------------------------------- errors */
const char* dg_status_string(dg_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* dg_last_error(void);

/* ---------------------------------------------------------------- model */
/* Most canvases one dg_generate_block call runs (its stop-flag slots are
 * allocated with the model). */
#define DG_MAX_LOOP_BATCH 4096

/* Validates the configuration and copies the weight pointer table.  Also
 * allocates the block loop's only host resources, once: two events and
 * 2 x DG_MAX_LOOP_BATCH int32 stop flags in pinned host memory (hipHostMalloc),
 * freed by dg_model_destroy; dg_generate_block reports DG_ERR_HIP when they
 * could not be allocated (no usable device at creation).
 * DG_ERR_SHAPE on unsupported shapes (limits listed in dg_config);
 * DG_ERR_DTYPE on an unknown dtype or expert_dtype, DG_ERR_UNSUPPORTED for
 * FP8 experts outside their limits, DG_ERR_ARG when their scales are
 * missing. */
dg_status dg_model_create(const dg_config* cfg, const dg_weights* w, dg_model** out);
void dg_model_destroy(dg_model* m);

/* Blocked layout (bf16 models with d_model % 256 == 0 and vocab % 128 == 0):
 * a matrix [R][K] is stored as tiles of 256 rows, each tile's K in stages of
 * 32 values; one stage of one tile (256 x 32 values, 16 KiB) is contiguous,
 * element (r, k) at ((r/256 * K/32 + k/32) * 256 + r%256) * 32 + k%32, with R
 * padded to a multiple of 256.  The vocabulary products stream their weight
 * one contiguous block per stage: at one canvas per call they are bound by
 * that weight stream (this implementation's own measurement of the head: HBM
 * traffic 1.03 x the algorithmic bytes, at AI 205 FLOP/B below the bf16
 * ridge), so whole 1 KiB runs per wave instruction matter.
 *
 * Writes the self-conditioning operand E^T [d][V] from d_embed [V][d]: in the
 * blocked layout for blocked models, else row-major.  d_out holds
 * vocab*d_model elements of the model dtype.  Errors: DG_ERR_ARG on NULL. */
dg_status dg_embed_transpose(const dg_model* m, const void* d_embed, void* d_out, void* stream);
/* Bytes of the blocked head operand of this model (E [V][d] in the blocked
 * layout, V padded to a multiple of 256), or 0 when the model's head reads
 * `embed` directly (not a blocked model). */
dg_status dg_embed_head_bytes(const dg_model* m, size_t* bytes);
/* Writes that operand from d_embed [V][d] into d_out (dg_embed_head_bytes
 * bytes); pass it as weights.embed_head.  DG_ERR_UNSUPPORTED for models that
 * are not blocked, DG_ERR_ARG on NULL. */
dg_status dg_embed_head(const dg_model* m, const void* d_embed, void* d_out, void* stream);

/* ---------------------------------------------------------------- KV cache */
/* Bytes of a KV cache for `batch` sequences of up to `capacity` positions:
 * K then V, each [n_layers][batch][n_kv_heads][capacity][head_dim] in the
 * model dtype, K after RoPE.  A denoising step needs capacity >= len + N
 * (the canvas K/V are staged in slots [len, len+N) without advancing len). */
dg_status dg_kv_bytes(const dg_model* m, int32_t batch, int32_t capacity, size_t* bytes);
/* Wraps caller memory (d_buf, >= dg_kv_bytes) as an empty cache (len = 0). */
dg_status dg_kv_create(const dg_model* m, int32_t batch, int32_t capacity, void* d_buf,
                       dg_kv** out);
void dg_kv_destroy(dg_kv* kv);
dg_status dg_kv_length(const dg_kv* kv, int32_t* len);
/* Rewinds (or advances) the valid length, e.g. to reuse an encoded prompt. */
dg_status dg_kv_set_length(dg_kv* kv, int32_t len);

/* 8-bit expert weights (youleyou.com article, "Deployment": the model ships
 * tuned for a 4-bit floating-point weight format on NVIDIA parts, to move
 * fewer bytes through the memory-bound experts; the CDNA4 analogue here is
 * OCP E4M3 with one scale per row).  Quantises d_src [rows][cols] (src_dtype
 * DG_F32 or DG_BF16) row by row: amax = max |x|, scale = amax / 448 in fp32
 * (1 for an all-zero row), code = E4M3 of the fp32 quotient x / scale, round
 * to nearest with ties to the even code, saturating at 448.  Writes d_scale
 * [rows] (fp32) and the rows*cols code bytes of d_q tiled in the order the
 * block-scaled expert kernels read their MFMA operands (rows % 16 == 0, cols %
 * 128 == 0): 16-row tiles, one after another; in a tile its 128-column steps,
 * one after another; a step is two 1-KiB halves (columns 0..63 and 64..127 of
 * the step), and in half h the 16 bytes at 16 * (16 g + r) are row r's
 * columns 64 h + 16 g .. +15.  An expert matrix [E][R][K] is rows = E*R,
 * cols = K.  DG_ERR_ARG on NULL or bad sizes, DG_ERR_DTYPE on another
 * src_dtype. */
dg_status dg_quantize_fp8(const void* d_src, int32_t src_dtype, int64_t rows, int32_t cols,
                          void* d_q, float* d_scale, void* stream);
/* 4-bit expert weights in the OCP microscaling format MXFP4 (same passage;
 * the closest CDNA4 format to the pages' 4-bit one; gfx950's block-scaled
 * matrix cores take it as stored).  Quantises d_src [rows][cols] (src_dtype
 * DG_F32 or DG_BF16, rows % 16 == 0, cols % 128 == 0) in blocks of 32
 * consecutive elements of a row: X = 2^(floor(log2(max |x|)) - 2), the
 * exponent clamped to [-127, 127] (an all-zero block takes 2^-127); code =
 * E2M1 of x / X, round to nearest with ties to the even code, magnitudes
 * above 6 giving 6.  Writes rows*cols/2 code bytes to d_codes (two codes a
 * byte, the even column in the low nibble) and rows*cols/32 E8M0 scale codes
 * (127 + log2 X) to d_scales, both tiled in the order the block-scaled expert
 * kernels read their MFMA operands: 16-row tiles, one after another; in a
 * tile its 128-column steps, one after another; a tile-step is 1 KiB of
 * codes, the 16 bytes at 16 * (16 g + r) holding row r's 32-column block g
 * of the step, and 64 scale codes, byte 16 g + r that block's.  An expert
 * matrix [E][R][K] is rows = E*R, cols = K.  DG_ERR_ARG on NULL or bad sizes,
 * DG_ERR_DTYPE on another src_dtype. */
dg_status dg_quantize_mxfp4(const void* d_src, int32_t src_dtype, int64_t rows, int32_t cols,
                            void* d_codes, uint8_t* d_scales, void* stream);

/* ---------------------------------------------------------------- workspace */
/* Bytes of scratch for every model call with up to `batch` sequences.
 * Prompts of any length are encoded in chunks that fit this workspace. */
dg_status dg_workspace_bytes(const dg_model* m, int32_t batch, size_t* bytes);
/* Bytes of scratch for dg_sample_update alone (no model needed). */
dg_status dg_sampler_workspace_bytes(int32_t batch, int32_t canvas, size_t* bytes);

/* ---------------------------------------------------------------- the path */

/* Causal encode of d_tokens [batch][n_tokens] (report-summary page, section 2;
 * youleyou.com article, "Architecture basis"): embeddings run through every
 * layer with causal attention over the cache plus the new tokens; K (after
 * RoPE) and V of every layer are appended at [len, len+n_tokens) and len
 * advances.  The last layer's MoE feeds no K/V and is skipped.
 * DG_ERR_CAPACITY if len + n_tokens > capacity. */
dg_status dg_encode_prompt(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_tokens,
                           int32_t n_tokens, void* d_ws, size_t ws_bytes, void* stream);

/* One denoiser forward over canvases d_canvas [batch][N] (report-summary
 * page, sections 2 and 5): h0 = E[x] + s W_sc^T with s = softmax(prev) E
 * (s = 0 when d_prev_logits is NULL); per layer pre-norm bidirectional
 * attention over [cache ; canvas] and top-k SwiGLU MoE; logits =
 * RMSNorm(h) E^T written to d_logits [batch][N][V] (fp32).
 * d_prev_stats [batch][N][4] are the per-position statistics dg_sample_update
 * wrote for d_prev_logits ({max, sum of exp(l - max), entropy, max-prob});
 * both are NULL or both are set.  The cache length is unchanged (canvas K/V
 * use slots [len, len+N), so capacity >= len + N is required). */
dg_status dg_denoise_step(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_canvas,
                          const float* d_prev_logits, const float* d_prev_stats,
                          float* d_logits, void* d_ws, size_t ws_bytes, void* stream);

/* dg_denoise_step whose self-conditioning uses the previous round's
 * distribution truncated to each position's top_k logits (what the sampler
 * used with params->top_k = top_k): s = sum_i p_i E[c_i] over the top_k
 * candidates c_i (value descending, ties to the lower index) with
 * p_i = e_i / S as the sampler defines them.  top_k = 0 is dg_denoise_step;
 * 1 <= top_k <= min(64, vocab) (DG_ERR_ARG otherwise).  d_prev_stats may be
 * NULL when top_k > 0. */
dg_status dg_denoise_step_topk(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_canvas,
                               const float* d_prev_logits, const float* d_prev_stats,
                               int32_t top_k, float* d_logits, void* d_ws, size_t ws_bytes,
                               void* stream);

/* Sampler update of step `step` (report-summary page, sections 1 and 4).
 * Model-free: reads fp32 logits [batch][N][V]; for every canvas b with
 * d_stop[b] == 0 it writes, per position,
 *   d_stats [b][i][4] = {max logit, sum exp(l - max), entropy H, max-prob}
 *   d_argmax[b][i]    = first index of the max logit (in: previous step's)
 *   d_lock[b][i]      = lock decision (rule in params)
 *   d_canvas[b][i]    = lock ? token drawn from softmax(l / T_step)
 *                            : uniform renoise token
 *   d_stop[b]         = 1 if the stop rule fires (or the budget is used up).
 * Canvases with d_stop[b] != 0 on entry are left untouched.  Logits must be
 * finite: a NaN or infinite logit makes its row's entropy NaN, and such a
 * canvas gets d_stop[b] = 2 with its canvas, argmax and locks left as they
 * were (its statistics are written), so the caller can tell a numerical
 * failure from a stop.  The binary32
 * arithmetic (statistics, draw, lock and stop) is fixed exactly, so results
 * are bit-reproducible and match the reference definition bit for bit.
 * Random numbers: Philox4x64-10, key (seed, 0), counter (step, b, i, 0).
 * params->top_k > 0 (<= 64, <= vocab): the statistics, argmax and draw use
 * each position's top_k logits only (value descending, ties to the lower
 * index; sums in that order; one inverse-CDF draw with word 0).
 * d_ws needs dg_sampler_workspace_bytes.  N <= 1024, vocab <= 524288. */
dg_status dg_sample_update(const dg_sampler_params* p, int32_t step, int32_t batch,
                           int32_t canvas, int32_t vocab, const float* d_logits,
                           int32_t* d_canvas, int32_t* d_argmax, uint8_t* d_lock,
                           float* d_stats, int32_t* d_stop, void* d_ws, size_t ws_bytes,
                           void* stream);

/* dg_sample_update for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same update with the same results, bit for bit, but no workspace
 * argument.  Its scratch (three int32 per row) is a static device array
 * inside the library, one per GPU, held until the process ends; the call
 * allocates nothing.  Limit: batch * canvas <= 65536 rows (DG_ERR_CAPACITY
 * otherwise, nothing launched).  The stream must belong to the calling
 * thread's current device.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (different streams or threads)
 * race and must not be issued; calls in one stream's order are safe. */
dg_status dg_sample_update_static(const dg_sampler_params* p, int32_t step, int32_t batch,
                                  int32_t canvas, int32_t vocab, const float* d_logits,
                                  int32_t* d_canvas, int32_t* d_argmax, uint8_t* d_lock,
                                  float* d_stats, int32_t* d_stop, void* stream);

/* dg_sample_update that also writes the next round's self-conditioning
 * operand (report-summary page, section 2: the model sees its previous
 * round's prediction; section 5: that costs a pass over the full
 * distributions), while it reads the logits anyway.  For every sampled row r
 * = b*N + i, d_probs receives the softmax numerators exp(l - M_r) exactly as
 * dg_stage_probs computes them, M_r = the largest of d_rowmax[r][0 ..
 * vocab/64) (dg_stage_head_rowmax writes them; it equals the statistics'
 * max), in the layout `blocked` selects as for dg_stage_probs: the same
 * bits dg_stage_probs writes.  All other
 * outputs are those of dg_sample_update.  vocab % 128 == 0 (DG_ERR_SHAPE
 * otherwise). */
dg_status dg_sample_update_probs(const dg_sampler_params* p, int32_t step, int32_t batch,
                                 int32_t canvas, int32_t vocab, const float* d_logits,
                                 int32_t* d_canvas, int32_t* d_argmax, uint8_t* d_lock,
                                 float* d_stats, int32_t* d_stop, const float* d_rowmax,
                                 int32_t blocked, void* d_probs, void* d_ws, size_t ws_bytes,
                                 void* stream);

/* Self-conditioning operand of T logit rows d_logits [T][vocab] with their
 * statistics d_stats [T][4] (as dg_sample_update writes them): d_probs =
 * the softmax numerators exp(l - stats[0]) as bf16; the division by
 * stats[1] follows the product with E inside the denoiser (report-summary
 * page, sections 2 and 5).  Computed in the sampler's row layout: for each
 * chunk with max m_c, E(l - m_c) * E(m_c - stats[0]) in binary32, E the
 * sampler's exp (so the row pass of dg_sample_update_probs, which already
 * holds E(l - m_c), writes the same bits).  blocked != 0: 64-wide blocks,
 * element (r, v) at ((r/256 * vocab/64 + v/64) * 256 + r%256) * 64 + v%64
 * over T rows padded to 256 (vocab % 64 == 0; one row's 64 values are one
 * 128-byte line), else row-major [T][vocab].  vocab % 4 == 0.  Model-free;
 * d_probs is caller-owned device memory. */
dg_status dg_stage_probs(int32_t T, int32_t vocab, int32_t blocked, const float* d_logits,
                         const float* d_stats, void* d_probs, void* stream);

/* Canvas initialisation: d_canvas [batch][N] = uniform tokens from Philox
 * counter (block_index, b, i, 1), key (seed, 0) (report-summary page,
 * section 1: the block starts as random tokens). */
dg_status dg_canvas_init(uint64_t seed, int32_t block_index, int32_t batch, int32_t canvas,
                         int32_t vocab, int32_t* d_canvas, void* stream);

/* Block commit (akiraxclaw.com blog, "memory, not compute"): causal encode of
 * the finished block d_block [batch][N] appended to the cache; len += N. */
dg_status dg_commit_block(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_block,
                          void* d_ws, size_t ws_bytes, void* stream);

/* One block of block-autoregressive generation: canvas init, up to
 * params->max_steps rounds of dg_denoise_step + dg_sample_update (self-
 * conditioned on the previous round if params->selfcond_on), stop per
 * canvas, block = the last round's argmax, then dg_commit_block.
 * d_block_out [batch][N]; h_steps_out [batch] receives the rounds each canvas
 * ran.  Waits on the stream once per round to read the stop flags.  A canvas
 * whose logits turn non-finite stops in that round (dg_sample_update's
 * d_stop = 2); the others run on, d_block_out and h_steps_out are written,
 * the block is NOT committed and the call returns DG_ERR_NONFINITE.
 * DG_ERR_CAPACITY if batch > DG_MAX_LOOP_BATCH.  The call allocates nothing.  For
 * blocked models with weights.embed_head the rounds run as
 * dg_stage_head_rowmax + dg_sample_update_probs, so the next round's
 * self-conditioning operand comes out of the sampler's pass over the logits
 * (the same bits as the separate pass dg_denoise_step makes).
 * d_ws needs dg_generate_workspace_bytes. */
dg_status dg_generate_workspace_bytes(const dg_model* m, int32_t batch, size_t* bytes);
dg_status dg_generate_block(dg_model* m, dg_kv* kv, int32_t batch, const dg_sampler_params* p,
                            int32_t block_index, int32_t* d_block_out, int32_t* h_steps_out,
                            void* d_ws, size_t ws_bytes, void* stream);
/* dg_generate_block that also records the per-round quantities the
 * report-summary page's section 4 describes the loop by (the mean-entropy
 * trajectory that the stop rule watches, and how many positions are locked):
 * d_trace [params->max_steps][batch][2] float, caller-owned device memory;
 * entry [t][b] = (mean entropy of canvas b's round-t logits, i.e. the value
 * the stop rule tests, and the number of its positions locked after round t)
 * for every round t < h_steps_out[b] that the canvas ran; (NaN, 0) for the
 * round in which a canvas's logits turned non-finite; entries of rounds a
 * canvas did not run are not written.  NULL d_trace is DG_ERR_ARG. */
dg_status dg_generate_block_trace(dg_model* m, dg_kv* kv, int32_t batch,
                                  const dg_sampler_params* p, int32_t block_index,
                                  int32_t* d_block_out, int32_t* h_steps_out, float* d_trace,
                                  void* d_ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- retained AR mode */
/* Report-summary page, section 7: the diffusion model keeps its
 * autoregressive starting point's architecture, so the same weights run as an
 * ordinary causal language model; section 5 describes that mode's step (one
 * new token per step over the cached history).
 *
 * One decode step: d_tokens [batch] (ids in [0, vocab)) at position len of
 * every sequence.  Every layer runs causal attention over the cache [0, len]
 * (the token's K/V written to slot len) and its MoE; then the final norm and
 * the tied head: d_logits [batch][vocab] fp32, 16-byte aligned.  len += 1.
 * To continue a prompt of P tokens, encode its first P - 1 with
 * dg_encode_prompt and decode the last one.  d_ws needs
 * dg_workspace_bytes(batch).  Errors: DG_ERR_SHAPE if batch != the cache's,
 * DG_ERR_CAPACITY if the cache is full (nothing launched). */
dg_status dg_ar_decode_step(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_tokens,
                            float* d_logits, void* d_ws, size_t ws_bytes, void* stream);
/* Greedy choice: d_out[r] = the index of row r's largest logit, ties to the
 * lower index (NaN entries never win; an all-NaN row gives 0).
 * d_logits [rows][vocab] fp32, 16-byte aligned. */
dg_status dg_argmax_rows(int32_t rows, int32_t vocab, const float* d_logits, int32_t* d_out,
                         void* stream);
/* Greedy decoding of n_new tokens per sequence: step t decodes the previous
 * token (d_first [batch] at t = 0, else d_out[b][t-1]) with
 * dg_ar_decode_step and writes the greedy choice of its logits to
 * d_out [batch][n_new] (row-major).  d_logits [batch][vocab] is scratch that
 * holds the last step's logits on return.  len += n_new.  Errors as
 * dg_ar_decode_step; DG_ERR_CAPACITY if len + n_new exceeds the capacity. */
dg_status dg_ar_generate(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_first,
                         int32_t n_new, int32_t* d_out, float* d_logits, void* d_ws,
                         size_t ws_bytes, void* stream);

/* -------------------------------------------------- training-side forward */
/* Report-summary page, section 1: training replaces a random share of a
 * text's tokens (from none to all) by junk and asks for the originals;
 * section 3: the supervised stage does this at varying degrees and learns
 * from the gap between prediction and original.  The forward pass only (no
 * gradients).
 *
 * Multinomial corruption: d_out[b][i] = uniform_token(word 1, vocab) if
 * uniform(word 0) < d_rate[b], else d_clean[b][i], with the Philox4x64-10
 * block of counter (step, b, i, 2), key (seed, 0) (the sampler's uniform and
 * uniform_token).  d_rate [batch] fp32 in [0, 1]; d_clean, d_out
 * [batch][canvas] int32 (may not alias). */
dg_status dg_corrupt(uint64_t seed, int32_t step, int32_t batch, int32_t canvas, int32_t vocab,
                     const float* d_rate, const int32_t* d_clean, int32_t* d_out, void* stream);
/* Cross-entropy of each row of d_logits [rows][vocab] fp32 at d_target[row]:
 * d_loss[row] = L(S) - (l[target] - m), m and S the row's max and sum of
 * E(l - m) as the sampler computes them (binary32, bit-exact with its
 * statistics); NaN for a target outside [0, vocab).  d_mean (optional, one
 * float) = the sequential binary32 sum of the losses in row order / rows.
 * vocab <= 2^19. */
dg_status dg_xent(int32_t rows, int32_t vocab, const float* d_logits, const int32_t* d_target,
                  float* d_loss, float* d_mean, void* stream);
/* Training-side forward of the canvases d_clean [batch][N] over the cached
 * context (which is not modified): dg_corrupt into d_corrupted [batch][N],
 * one denoiser forward of the corrupted canvases with no self-conditioning
 * input (d_logits [batch][N][vocab] fp32), and dg_xent at the clean tokens
 * (d_loss [batch][N], d_mean optional).  d_ws needs dg_workspace_bytes(batch).
 * Errors: DG_ERR_SHAPE if batch != the cache's; DG_ERR_CAPACITY if
 * len + N exceeds the capacity (nothing launched). */
dg_status dg_train_forward(dg_model* m, dg_kv* kv, int32_t batch, const int32_t* d_clean,
                           const float* d_rate, uint64_t seed, int32_t step, int32_t* d_corrupted,
                           float* d_logits, float* d_loss, float* d_mean, void* d_ws,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- stages */
/* The step's stages, exposed so each can be driven and checked on its own.
 * T = number of tokens; h buffers are fp32 [T][d] residual streams. */

/* Denoiser input: d_h [batch*N][d] = E[canvas] + (softmax(prev) E) W_sc^T. */
dg_status dg_stage_input(dg_model* m, int32_t batch, const int32_t* d_canvas,
                         const float* d_prev_logits, const float* d_prev_stats, float* d_h,
                         void* d_ws, size_t ws_bytes, void* stream);
/* dg_stage_input with the self-conditioning truncated to each position's
 * top_k previous logits, as dg_denoise_step_topk computes it (report-summary
 * page, section 9: top-k truncation): s = sum_i p_i E[c_i] over the top_k
 * candidates.  1 <= top_k <= min(64, vocab) (DG_ERR_ARG otherwise). */
dg_status dg_stage_input_topk(dg_model* m, int32_t batch, const int32_t* d_canvas,
                              const float* d_prev_logits, int32_t top_k, float* d_h, void* d_ws,
                              size_t ws_bytes, void* stream);
/* Attention half-block of `layer` for n new tokens per sequence at positions
 * [len, len+n): RMSNorm, Q/K/V, RoPE, K/V written to cache slots [len, len+n),
 * attention (causal != 0: each query sees keys <= its position; causal == 0:
 * every query sees all len+n keys), output projection, residual into d_h
 * [batch*n][d].  The cache length is not changed. */
dg_status dg_stage_attention(dg_model* m, dg_kv* kv, int32_t layer, int32_t batch, int32_t n,
                             int32_t causal, float* d_h, void* d_ws, size_t ws_bytes,
                             void* stream);
/* MoE half-block of `layer` over T tokens: RMSNorm, router, top-k, SwiGLU
 * experts, gate-weighted sum, residual into d_h [T][d].  If d_route is not
 * NULL it receives the chosen experts [T][top_k] (selection order) and
 * d_gates [T][top_k] the gates. */
dg_status dg_stage_moe(dg_model* m, int32_t layer, int32_t T, float* d_h, int32_t* d_route,
                       float* d_gates, void* d_ws, size_t ws_bytes, void* stream);
/* Head: d_logits [T][V] = RMSNorm(d_h) E^T (fp32), in the launch configuration
 * a step over ceil(T / N) canvases uses; d_ws needs
 * dg_workspace_bytes(ceil(T / N)) (DG_ERR_CAPACITY otherwise). */
dg_status dg_stage_head(dg_model* m, int32_t T, const float* d_h, float* d_logits, void* d_ws,
                        size_t ws_bytes, void* stream);
/* The head as the block loop runs it: dg_stage_head, and d_rowmax [T][V/64]
 * = the largest logit of each row in each 64-column slab, taken from the
 * product's registers before the logits are read again.  Blocked models with
 * weights.embed_head only (DG_ERR_UNSUPPORTED otherwise); d_ws needs
 * dg_workspace_bytes(ceil(T / N)) (DG_ERR_CAPACITY otherwise). */
dg_status dg_stage_head_rowmax(dg_model* m, int32_t T, const float* d_h, float* d_logits,
                               float* d_rowmax, void* d_ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- timers */
/* Kernel timers: when enabled, the library records a pair of HIP events on
 * the launch stream around every launch of the selected kernels, so a caller
 * can measure each kernel's average duration inside its own timed region.
 * Process-wide state; enable/read from one thread. */
typedef enum {
    DG_TIMER_HEAD_GEMM = 0,      /* logits = RMSNorm(h) E^T (the GEMM launch)        */
    DG_TIMER_SELFCOND_GEMM = 1,  /* softmax(prev) E split-K product                 */
    DG_TIMER_MOE_GATEUP = 2,     /* grouped SwiGLU gate/up expert GEMM               */
    DG_TIMER_MOE_DOWN = 3,       /* grouped down-projection expert GEMM              */
    DG_TIMER_ATTENTION = 4,      /* attention (+ split merge)                        */
    DG_TIMER_SAMPLER = 5,        /* per-row sampler kernel + per-canvas kernel       */
    DG_TIMER_COUNT = 6
} dg_timer_id;
/* Bit i of mask enables timer i; clears all recorded events.  0 disables. */
dg_status dg_timer_enable(uint32_t mask);
/* Waits for the recorded events of timer `id` and returns the summed
 * duration (ms) and number of launches since the last dg_timer_enable. */
dg_status dg_timer_read(int32_t id, double* total_ms, int64_t* launches);

/* ------------------------------------------------------- calibration */
/* Microbenchmark peaks of the current device, for reporting beside the
 * published ones; no step of the denoising path uses them.  Runs two probe
 * kernels on `stream` and waits for them:
 *   *hbm_read_gbs     = bytes per second of a read-only stream over d_buf
 *                       (non-temporal 16-byte loads, 8 workgroups a CU,
 *                       5 passes timed after one untimed);
 *   *mfma_bf16_tflops = FLOP/s of independent v_mfma_f32_16x16x32_bf16
 *                       (four accumulators a wave, eight waves a SIMD).
 * d_buf is caller-owned device memory of buf_bytes >= 256 MiB plus a few MB
 * (DG_ERR_CAPACITY otherwise); its contents are overwritten.  DG_ERR_HIP if
 * a launch or event call fails. */
dg_status dg_measure_peaks(void* d_buf, size_t buf_bytes, void* stream, double* hbm_read_gbs,
                           double* mfma_bf16_tflops);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
