"""Seeded synthetic inputs: model shapes, random-init weights and uniform tokens.

This module holds no arithmetic of the method: it only draws numbers.  Both the
HIP path (through the tests and the benchmark) and the CPU oracle consume what
it produces; neither side imports the other.

Recipe (the pages publish no weights, datasets or prompts):
  * weights ~ N(0, 0.02^2) from numpy.random.default_rng(seed), drawn in the
    order embed, w_sc, then per layer wq, wk, wv, wo, w_router, w_gate, w_up,
    w_down; RMSNorm scales are ones;
  * bf16 models round each weight once, to nearest-even, and both sides use
    the rounded values;
  * prompt tokens are uniform in [0, V) from default_rng([seed, 1]).
"""
from __future__ import annotations

import numpy as np

# Model shapes.  "canvas" = 256 tokens refined in parallel; 128 experts with 8
# active; vocabulary 262144 for the full head.
SHAPES = {
    # 1-layer tiny denoiser in fp32: parity at 1e-4
    "tiny": dict(n_layers=1, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64, n_experts=8,
                 top_k=2, d_ff=512, vocab=1024, canvas=256, dtype="f32", prompt=32, batch=1,
                 max_steps=4),
    # one denoiser layer at production width, bf16, prompt KV 2048, full vocab head
    "layer": dict(n_layers=1, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128,
                  n_experts=128, top_k=8, d_ff=768, vocab=262144, canvas=256, dtype="bf16",
                  prompt=2048, batch=1, max_steps=48),
    # the same layer with 8-bit (E4M3, per-row scale) expert weights
    "layer_fp8": dict(n_layers=1, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128,
                      n_experts=128, top_k=8, d_ff=768, vocab=262144, canvas=256, dtype="bf16",
                      expert_dtype="fp8", prompt=2048, batch=1, max_steps=48),
    # the same layer with MXFP4 expert weights
    "layer_mxfp4": dict(n_layers=1, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128,
                        n_experts=128, top_k=8, d_ff=768, vocab=262144, canvas=256, dtype="bf16",
                        expert_dtype="mxfp4", prompt=2048, batch=1, max_steps=48),
    # 30 such layers, prompt 4096
    # (its sampler: temperature 1, lock where the max-probability exceeds 0.9)
    "stack": dict(n_layers=30, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128,
                  n_experts=128, top_k=8, d_ff=768, vocab=262144, canvas=256, dtype="bf16",
                  prompt=4096, batch=1, max_steps=48,
                  sampler=dict(lock_rule=0, lock_theta=0.9, temp_start=1.0, temp_end=1.0)),
    # 8 canvases with 8192-token prompts each
    "batched": dict(n_layers=30, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128,
                    n_experts=128, top_k=8, d_ff=768, vocab=262144, canvas=256, dtype="bf16",
                    prompt=8192, batch=8, max_steps=48, stop_tau=0.05),
    # long prompt, 8 consecutive blocks committed to the cache
    "long": dict(n_layers=30, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128,
                 n_experts=128, top_k=8, d_ff=768, vocab=262144, canvas=256, dtype="bf16",
                 prompt=32768, batch=1, max_steps=48, blocks=8),
}

MODEL_KEYS = ("n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
              "d_ff", "vocab", "canvas")


def model_config(name_or_shape, **over) -> dict:
    """Model hyper-parameters (shape dict plus rope/norm defaults)."""
    base = dict(SHAPES[name_or_shape]) if isinstance(name_or_shape, str) else dict(name_or_shape)
    cfg = {k: base[k] for k in MODEL_KEYS}
    cfg.update(dtype=base.get("dtype", "bf16"), rope_on=1, rope_theta=10000.0, rms_eps=1e-6,
               selfcond_on=1)
    if base.get("expert_dtype"):
        cfg["expert_dtype"] = base["expert_dtype"]
    cfg.update(over)
    # the oracle's names
    cfg["d"] = cfg["d_model"]
    return cfg


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def make_weights(cfg: dict, seed: int = 0, std: float = 0.02, random_norms: bool = False) -> dict:
    """Random-init weights as float32 arrays ([out, in] per linear map).
    bf16 models get bf16-representable values."""
    rng = np.random.default_rng(seed)
    d, V = cfg["d_model"], cfg["vocab"]
    Hq, Hkv, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    E, F = cfg["n_experts"], cfg["d_ff"]
    rnd = round_bf16 if cfg["dtype"] == "bf16" else (lambda a: a)

    def draw(*shape):
        return rnd(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))

    def norm():
        if random_norms:
            return (1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32)).astype(np.float32)
        return np.ones(d, dtype=np.float32)

    W = {"embed": draw(V, d), "w_sc": draw(d, d)}
    layers = []
    for _ in range(cfg["n_layers"]):
        lw = {"attn_norm": norm()}
        lw["wq"] = draw(Hq * dh, d)
        lw["wk"] = draw(Hkv * dh, d)
        lw["wv"] = draw(Hkv * dh, d)
        lw["wo"] = draw(d, Hq * dh)
        lw["moe_norm"] = norm()
        lw["w_router"] = draw(E, d)
        lw["w_gate"] = draw(E, F, d)
        lw["w_up"] = draw(E, F, d)
        lw["w_down"] = draw(E, d, F)
        layers.append(lw)
    W["layers"] = layers
    W["final_norm"] = norm()
    return W


def make_tokens(V: int, shape, seed: int = 0, stream: int = 1) -> np.ndarray:
    """Uniform tokens in [0, V) as int32."""
    rng = np.random.default_rng([seed, stream])
    return rng.integers(0, V, size=shape, dtype=np.int64).astype(np.int32)


def make_logits(shape, seed: int = 0, sigma: float = 0.9) -> np.ndarray:
    """Gaussian logits N(0, sigma^2) as float32 (a stand-in for a random-init head)."""
    rng = np.random.default_rng([seed, 2])
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def to_float64(W: dict) -> dict:
    """The same weights as float64 (for the oracle)."""
    out = {k: np.asarray(v, dtype=np.float64) for k, v in W.items() if k != "layers"}
    out["layers"] = [{k: np.asarray(v, dtype=np.float64) for k, v in lw.items()}
                     for lw in W["layers"]]
    return out


def default_sampler_params(**over) -> dict:
    """Sampler knobs.  Defaults are the values the report-summary page gives
    in its sampler section: cumulative-entropy locking at 0.1, temperature
    0.8 -> 0.4, stop at mean entropy < 0.005 with an unchanged most likely
    sequence, at most 48 rounds."""
    p = dict(lock_rule=1, lock_theta=0.1, temp_start=0.8, temp_end=0.4, stop_tau=0.005,
             require_stable=1, max_steps=48, seed=0, selfcond_on=1, top_k=0)
    p.update(over)
    return p
