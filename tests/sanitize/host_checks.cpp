// Host-side checks of the library's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every call here returns before any GPU work
// (argument validation, shape and dtype checks, size queries, handles), so
// the run needs no GPU.  Exit code 0 when every status is the documented one.
#include <cstdio>
#include <cstring>
#include <vector>

#include "dg.h"

static int failures = 0;

static void expect(dg_status got, dg_status want, const char* what) {
    if (got != want) {
        std::fprintf(stderr, "%s: status %d (%s), expected %d: %s\n", what, (int)got,
                     dg_status_string(got), (int)want, dg_last_error());
        ++failures;
    }
}

static dg_config base_config() {
    dg_config c;
    std::memset(&c, 0, sizeof c);
    c.n_layers = 2;
    c.d_model = 256;
    c.n_heads = 4;
    c.n_kv_heads = 2;
    c.head_dim = 64;
    c.n_experts = 8;
    c.top_k = 2;
    c.d_ff = 256;
    c.vocab = 1024;
    c.canvas = 256;
    c.dtype = DG_BF16;
    c.rope_on = 1;
    c.rope_theta = 10000.f;
    c.rms_eps = 1e-6f;
    return c;
}

int main() {
    // the status strings and the per-thread error text
    for (int s = DG_OK; s <= DG_ERR_UNSUPPORTED; ++s)
        if (!dg_status_string((dg_status)s)) ++failures;
    if (!dg_last_error()) ++failures;

    // weights: addresses that are never dereferenced on the host
    void* fake = (void*)0x1000;
    std::vector<dg_layer_weights> lw(2);
    for (auto& l : lw) {
        std::memset(&l, 0, sizeof l);
        l.attn_norm = (const float*)fake;
        l.wq = l.wk = l.wv = l.wo = fake;
        l.moe_norm = (const float*)fake;
        l.w_router = l.w_gate = l.w_up = l.w_down = fake;
    }
    dg_weights w;
    std::memset(&w, 0, sizeof w);
    w.embed = w.embed_t = w.w_sc = fake;
    w.final_norm = (const float*)fake;
    w.layers = lw.data();

    dg_model* m = nullptr;
    expect(dg_model_create(nullptr, &w, &m), DG_ERR_ARG, "create without config");
    dg_config c = base_config();
    c.dtype = 9;
    expect(dg_model_create(&c, &w, &m), DG_ERR_DTYPE, "unknown dtype");
    c = base_config();
    c.head_dim = 96;
    expect(dg_model_create(&c, &w, &m), DG_ERR_SHAPE, "head_dim 96");
    c = base_config();
    c.top_k = 9;
    expect(dg_model_create(&c, &w, &m), DG_ERR_SHAPE, "top_k > n_experts");
    c = base_config();
    c.expert_dtype = DG_FP8_E4M3;
    expect(dg_model_create(&c, &w, &m), DG_ERR_ARG, "fp8 experts without scales");
    c = base_config();
    expect(dg_model_create(&c, &w, &m), DG_OK, "create");

    size_t bytes = 0;
    expect(dg_workspace_bytes(m, 2, &bytes), DG_OK, "workspace bytes");
    if (bytes == 0) ++failures;
    expect(dg_generate_workspace_bytes(m, 2, &bytes), DG_OK, "generate workspace bytes");
    expect(dg_kv_bytes(m, 2, 600, &bytes), DG_OK, "kv bytes");
    expect(dg_embed_head_bytes(m, &bytes), DG_OK, "embed head bytes");
    expect(dg_sampler_workspace_bytes(2, 256, &bytes), DG_OK, "sampler workspace bytes");
    expect(dg_sampler_workspace_bytes(0, 256, &bytes), DG_ERR_ARG, "sampler workspace batch 0");

    dg_kv* kv = nullptr;
    expect(dg_kv_create(m, 2, 600, fake, &kv), DG_OK, "kv create");
    expect(dg_kv_set_length(kv, 601), DG_ERR_CAPACITY, "kv length past capacity");
    expect(dg_kv_set_length(kv, 500), DG_OK, "kv length");
    int32_t len = 0;
    expect(dg_kv_length(kv, &len), DG_OK, "kv length read");
    if (len != 500) ++failures;

    // argument errors are returned before anything is launched
    int32_t* tok = (int32_t*)fake;
    float* lg = (float*)fake;
    expect(dg_encode_prompt(m, kv, 2, tok, 200, fake, 1 << 30, nullptr), DG_ERR_CAPACITY,
           "encode past capacity");
    expect(dg_encode_prompt(m, kv, 3, tok, 10, fake, 1 << 30, nullptr), DG_ERR_SHAPE,
           "encode with the wrong batch");
    expect(dg_denoise_step(m, kv, 2, tok, lg, nullptr, lg, fake, 1 << 30, nullptr), DG_ERR_ARG,
           "denoise with logits but no statistics");
    expect(dg_denoise_step(m, kv, 2, tok, nullptr, nullptr, lg, fake, 16, nullptr),
           DG_ERR_CAPACITY, "denoise with a small workspace");
    dg_sampler_params p;
    std::memset(&p, 0, sizeof p);
    p.lock_rule = DG_LOCK_CUMENT;
    p.lock_theta = 0.1f;
    p.temp_start = 0.8f;
    p.temp_end = 0.4f;
    p.stop_tau = 0.005f;
    p.require_stable = 1;
    p.max_steps = 48;
    expect(dg_sample_update(&p, 0, 2, 256, 1024, lg, tok, tok, (uint8_t*)fake, lg, tok, fake, 16,
                            nullptr),
           DG_ERR_CAPACITY, "sampler with a small workspace");
    p.top_k = 65;
    expect(dg_sample_update(&p, 0, 2, 256, 1024, lg, tok, tok, (uint8_t*)fake, lg, tok, fake,
                            1 << 20, nullptr),
           DG_ERR_ARG, "sampler top_k 65");
    p.top_k = 0;
    p.temp_start = 0.f;
    expect(dg_sample_update(&p, 0, 2, 256, 1024, lg, tok, tok, (uint8_t*)fake, lg, tok, fake,
                            1 << 20, nullptr),
           DG_ERR_ARG, "sampler temperature 0");
    p.temp_start = 0.8f;
    expect(dg_sample_update_static(&p, 0, 65, 1024, 8, lg, tok, tok, (uint8_t*)fake, lg, tok,
                                   nullptr),
           DG_ERR_CAPACITY, "static sampler above its rows");
    expect(dg_generate_block(m, kv, 3, &p, 0, tok, tok, fake, 1 << 30, nullptr), DG_ERR_SHAPE,
           "generate with the wrong batch");
    expect(dg_stage_moe(m, 2, 10, lg, nullptr, nullptr, fake, 1 << 30, nullptr), DG_ERR_ARG,
           "MoE stage of a layer past the last");
    expect(dg_ar_decode_step(m, kv, 2, nullptr, lg, fake, 1 << 30, nullptr), DG_ERR_ARG,
           "decode without tokens");
    expect(dg_argmax_rows(1, 8, (const float*)0x1004, tok, nullptr), DG_ERR_ARG,
           "argmax of unaligned logits");
    expect(dg_xent(0, 8, lg, tok, lg, nullptr, nullptr), DG_ERR_ARG, "cross-entropy of no rows");
    expect(dg_quantize_mxfp4(fake, DG_F32, 4, 96, fake, (uint8_t*)fake, nullptr), DG_ERR_ARG,
           "MXFP4 columns not a multiple of 64");
    expect(dg_timer_read(99, nullptr, nullptr), DG_ERR_ARG, "timer id out of range");

    dg_kv_destroy(kv);
    dg_model_destroy(m);
    if (failures) std::fprintf(stderr, "%d host check(s) failed\n", failures);
    else std::printf("host checks ok\n");
    return failures ? 1 : 0;
}
