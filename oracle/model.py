"""Plain float64 CPU oracle of the denoiser forward pass (numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.  It shares no code
with the HIP library.  Every function is the textbook definition written out,
with numpy's matmul as the only library primitive.

What the pages fix, and where:
  * report-summary page (animattoys.com), section 2: one set of weights runs
    with *causal* attention over the prompt (the context encoder) and with
    *bidirectional* attention over the 256-token canvas; a mixture of 128
    experts with 8 active per token; a self-conditioning input that lets the
    model see its previous round's prediction;
  * youleyou.com article, "Architecture basis": the causal encoder stores the
    prompt in the KV cache; every canvas position sees all canvas positions
    and the cached context;
  * akiraxclaw.com blog, "memory, not compute": a finished canvas is encoded
    into the KV cache and the next canvas starts (block-autoregressive);
  * report-summary page, section 5: the sampling cost includes the full
    distribution of every canvas position, the self-conditioning vector
    matrix product and a softmax over the whole vocabulary.
Everything else (pre-norm RMSNorm, rotate-half RoPE, SwiGLU experts, softmax
over the selected router logits, a single d x d self-conditioning projection
of the expected embedding, tied output head) is the plainest reading the pages
support; each is named where it is used below.

Weight layout (all float64 here): every linear map is stored as
[out_features, in_features] and applied as x @ W.T.
  embed [V, d]; w_sc [d, d]; final_norm [d]
  per layer: attn_norm [d], wq [Hq*dh, d], wk [Hkv*dh, d], wv [Hkv*dh, d],
  wo [d, Hq*dh], moe_norm [d], w_router [E, d], w_gate [E, F, d],
  w_up [E, F, d], w_down [E, d, F]
"""
from __future__ import annotations

import numpy as np

from . import quant


# ---------------------------------------------------------------- primitives

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding.  x [n, H, dh], pos [n] absolute positions.
    Pair (j, j + dh/2) is rotated by angle pos * theta^(-2j/dh)."""
    n, H, dh = x.shape
    half = dh // 2
    j = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]  # [n, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Grouped-query attention, explicit softmax per query row.
    q [n, Hq, dh]; k, v [m, Hkv, dh]; allowed [n, m] bool (True = key visible).
    Query head h reads kv head h // (Hq / Hkv); scores scaled by 1/sqrt(dh)."""
    n, Hq, dh = q.shape
    m, Hkv, _ = k.shape
    group = Hq // Hkv
    out = np.zeros((n, Hq, dh), dtype=np.float64)
    scale = 1.0 / np.sqrt(dh)
    for h in range(Hq):
        kh = k[:, h // group, :]
        vh = v[:, h // group, :]
        s = (q[:, h, :] @ kh.T) * scale                     # [n, m]
        s = np.where(allowed, s, -np.inf)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ vh
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def route(z: np.ndarray, top_k: int):
    """Top-k experts per token by router logit, ties to the lower expert id,
    listed in selection order; gates = softmax over the selected logits."""
    T, E = z.shape
    idx = np.zeros((T, top_k), dtype=np.int64)
    for t in range(T):
        # stable sort on -z keeps the lower id first among equal logits
        idx[t] = np.argsort(-z[t], kind="stable")[:top_k]
    zs = np.take_along_axis(z, idx, axis=1)
    g = np.exp(zs - zs.max(axis=1, keepdims=True))
    g = g / g.sum(axis=1, keepdims=True)
    return idx, g


def moe(u: np.ndarray, lw: dict, top_k: int, idx: np.ndarray | None = None,
        act_mx8: bool = False):
    """Sparse MoE of normalised tokens u [T, d]: router logits z = u W_r^T,
    top-k routing, y_t = sum_e g_e * W_down,e (silu(W_gate,e u) * (W_up,e u)).
    If idx is given it replaces the router's choice (gates still softmax of
    the chosen logits).  act_mx8 (the quantised experts): each expert
    product's input is rounded to MXFP8 along its features first -- u for
    gate and up (the router still sees u itself), silu(gate) * up for down,
    before the routing weight (oracle.quant.mx8_round).  Returns (y [T, d],
    idx, gates, z)."""
    z = u @ lw["w_router"].T
    if idx is None:
        idx, g = route(z, top_k)
    else:
        zs = np.take_along_axis(z, idx, axis=1)
        g = np.exp(zs - zs.max(axis=1, keepdims=True))
        g = g / g.sum(axis=1, keepdims=True)
    T, d = u.shape
    y = np.zeros((T, d), dtype=np.float64)
    xin = quant.mx8_round(u) if act_mx8 else u
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        x = xin[rows]
        a = silu(x @ lw["w_gate"][e].T) * (x @ lw["w_up"][e].T)
        if act_mx8:
            a = quant.mx8_round(a)
        y[rows] += g[rows, slots][:, None] * (a @ lw["w_down"][e].T)
    return y, idx, g, z


def act_mx8(cfg: dict) -> bool:
    """Whether the model's expert products take MXFP8 activations: the
    quantised expert formats (E4M3 per-row and MXFP4 weights)."""
    return cfg.get("expert_dtype") in ("fp8", "mxfp4")


# ---------------------------------------------------------------- KV cache

class KVCache:
    """Per layer: K (after RoPE) and V as [B, Hkv, length, dh] float64."""

    def __init__(self, cfg: dict, B: int):
        L, Hkv, dh = cfg["n_layers"], cfg["n_kv_heads"], cfg["head_dim"]
        self.k = [np.zeros((B, Hkv, 0, dh)) for _ in range(L)]
        self.v = [np.zeros((B, Hkv, 0, dh)) for _ in range(L)]
        self.length = 0

    def copy(self):
        c = KVCache.__new__(KVCache)
        c.k = [a.copy() for a in self.k]
        c.v = [a.copy() for a in self.v]
        c.length = self.length
        return c


# ---------------------------------------------------------------- layer

def attn_half(h: np.ndarray, lw: dict, cfg: dict, k_ctx: np.ndarray, v_ctx: np.ndarray,
              pos0: int, causal: bool):
    """Attention half-block of one sequence.
    h [n, d] residual stream of n new tokens at positions pos0..pos0+n-1;
    k_ctx, v_ctx [Hkv, pos0, dh] cached context.  Returns (h', k_new, v_new)
    with k_new, v_new [Hkv, n, dh] (K after RoPE)."""
    n, d = h.shape
    Hq, Hkv, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    u = rmsnorm(h, lw["attn_norm"], cfg["rms_eps"])
    q = (u @ lw["wq"].T).reshape(n, Hq, dh)
    k = (u @ lw["wk"].T).reshape(n, Hkv, dh)
    v = (u @ lw["wv"].T).reshape(n, Hkv, dh)
    pos = pos0 + np.arange(n)
    if cfg["rope_on"]:
        q = rope(q, pos, cfg["rope_theta"])
        k = rope(k, pos, cfg["rope_theta"])
    k_all = np.concatenate([k_ctx.transpose(1, 0, 2), k], axis=0)   # [pos0+n, Hkv, dh]
    v_all = np.concatenate([v_ctx.transpose(1, 0, 2), v], axis=0)
    m = pos0 + n
    if causal:
        # query at absolute position p sees keys 0..p
        allowed = np.arange(m)[None, :] <= pos[:, None]
    else:
        # canvas: every query sees the whole context and the whole canvas
        allowed = np.ones((n, m), dtype=bool)
    o = attention(q, k_all, v_all, allowed).reshape(n, Hq * dh)
    h = h + o @ lw["wo"].T
    return h, k.transpose(1, 0, 2), v.transpose(1, 0, 2)


def moe_half(h: np.ndarray, lw: dict, cfg: dict, idx: np.ndarray | None = None):
    """MoE half-block: h + MoE(RMSNorm(h)).  Returns (h', idx, gates, z)."""
    u = rmsnorm(h, lw["moe_norm"], cfg["rms_eps"])
    y, idx, g, z = moe(u, lw, cfg["top_k"], idx, act_mx8(cfg))
    return h + y, idx, g, z


# ---------------------------------------------------------------- stack

def embed(tokens: np.ndarray, W: dict) -> np.ndarray:
    """Token embedding rows E[x] (no scaling)."""
    return W["embed"][np.asarray(tokens)]


def topk_candidates(row: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest entries of a logit row, by value descending,
    ties to the lower index (the sampler's top-k truncation); a NaN ranks
    above every number and NaNs tie among themselves."""
    row = np.asarray(row, dtype=np.float64)
    nan = np.isnan(row)
    order = np.lexsort((np.arange(row.size), -np.where(nan, 0.0, row), ~nan))
    return order[:min(K, row.size)]


def selfcond_vector(prev_logits: np.ndarray, W: dict, top_k: int = 0) -> np.ndarray:
    """Expected embedding under the previous round's T = 1 distribution:
    s = softmax(L_prev) E, per position.  prev_logits [..., V].  With top_k
    > 0 the distribution is truncated to each position's top_k logits and
    renormalised (report-summary page, section 9 (known limitations): top-k truncation)."""
    L = np.asarray(prev_logits, dtype=np.float64)
    if top_k <= 0:
        p = np.exp(L - L.max(axis=-1, keepdims=True))
        p = p / p.sum(axis=-1, keepdims=True)
        return p @ W["embed"]
    flat = L.reshape(-1, L.shape[-1])
    out = np.zeros((flat.shape[0], W["embed"].shape[1]))
    for r in range(flat.shape[0]):
        c = topk_candidates(flat[r], top_k)
        p = np.exp(flat[r, c] - flat[r, c[0]])
        out[r] = (p / p.sum()) @ W["embed"][c]
    return out.reshape(L.shape[:-1] + (W["embed"].shape[1],))


def denoiser_input(canvas: np.ndarray, W: dict, prev_logits: np.ndarray | None,
                   top_k: int = 0) -> np.ndarray:
    """h0 = E[x] + s W_sc^T, with s = 0 when there is no previous prediction."""
    h = embed(canvas, W)
    if prev_logits is not None:
        s = selfcond_vector(prev_logits, W, top_k)
        h = h + s @ W["w_sc"].T
    return h


def head(h: np.ndarray, W: dict, cfg: dict) -> np.ndarray:
    """Tied output head: logits = RMSNorm(h) E^T."""
    return rmsnorm(h, W["final_norm"], cfg["rms_eps"]) @ W["embed"].T


def encode(tokens: np.ndarray, W: dict, cfg: dict, cache: KVCache) -> None:
    """Causal encode of tokens [B, n] appended after cache.length; K/V of each
    layer are appended to the cache.  The last layer's MoE output feeds no
    K/V, so it is not computed."""
    tokens = np.asarray(tokens)
    B, n = tokens.shape
    pos0 = cache.length
    for b in range(B):
        h = embed(tokens[b], W)
        for li, lw in enumerate(W["layers"]):
            h, kn, vn = attn_half(h, lw, cfg, cache.k[li][b][:, :pos0], cache.v[li][b][:, :pos0],
                                  pos0, causal=True)
            if b == 0:
                cache.k[li] = np.concatenate(
                    [cache.k[li], np.zeros(cache.k[li].shape[:2] + (n, cfg["head_dim"]))], axis=2)
                cache.v[li] = np.concatenate(
                    [cache.v[li], np.zeros(cache.v[li].shape[:2] + (n, cfg["head_dim"]))], axis=2)
            cache.k[li][b, :, pos0:pos0 + n] = kn
            cache.v[li][b, :, pos0:pos0 + n] = vn
            if li + 1 < len(W["layers"]):
                h, _, _, _ = moe_half(h, lw, cfg)
    cache.length = pos0 + n


# ---------------------------------------------------------------- AR mode
# Report-summary page, section 7: the diffusion model keeps its autoregressive
# starting point's architecture, so the same weights also run as an ordinary
# causal language model.  Section 5 describes that mode's step: one new token
# per step, attending over the cached history.  Plainest reading: the same
# stack with causal attention for every layer, every layer's MoE, the final
# norm and the tied head on the new token; greedy decoding takes the largest
# logit.

def causal_logits(tokens: np.ndarray, W: dict, cfg: dict) -> np.ndarray:
    """Causal language-model forward of one sequence tokens [n] from an empty
    context: every layer with causal attention and its MoE, then the head.
    Returns float64 logits [n, V]; row t scores the token after position t."""
    tokens = np.asarray(tokens).reshape(-1)
    h = embed(tokens, W)
    empty = np.zeros((cfg["n_kv_heads"], 0, cfg["head_dim"]))
    for lw in W["layers"]:
        h, _, _ = attn_half(h, lw, cfg, empty, empty, 0, causal=True)
        h, _, _, _ = moe_half(h, lw, cfg)
    return head(h, W, cfg)


def ar_decode_step(tokens: np.ndarray, W: dict, cfg: dict, cache: KVCache) -> np.ndarray:
    """One decode step of B sequences: tokens [B] at position cache.length.
    Each layer appends the token's K/V to the cache, and every layer's MoE
    runs (the token's hidden state feeds the head).  Returns float64 logits
    [B, V]; the cache grows by one position."""
    tokens = np.asarray(tokens).reshape(-1)
    B = tokens.size
    pos0 = cache.length
    dh = cfg["head_dim"]
    for li in range(len(W["layers"])):
        cache.k[li] = np.concatenate([cache.k[li], np.zeros(cache.k[li].shape[:2] + (1, dh))],
                                     axis=2)
        cache.v[li] = np.concatenate([cache.v[li], np.zeros(cache.v[li].shape[:2] + (1, dh))],
                                     axis=2)
    out = np.zeros((B, W["embed"].shape[0]))
    for b in range(B):
        h = embed(tokens[b:b + 1], W)
        for li, lw in enumerate(W["layers"]):
            h, kn, vn = attn_half(h, lw, cfg, cache.k[li][b][:, :pos0], cache.v[li][b][:, :pos0],
                                  pos0, causal=True)
            cache.k[li][b, :, pos0:pos0 + 1] = kn
            cache.v[li][b, :, pos0:pos0 + 1] = vn
            h, _, _, _ = moe_half(h, lw, cfg)
        out[b] = head(h, W, cfg)[0]
    cache.length = pos0 + 1
    return out


def greedy_token(logits: np.ndarray) -> np.ndarray:
    """Greedy choice per row: the index of the largest logit, ties to the
    lower index; a NaN ranks above every number (numpy's argmax returns the
    first NaN of a row)."""
    return np.argmax(np.asarray(logits), axis=-1).astype(np.int32)


def ar_generate(first: np.ndarray, n_new: int, W: dict, cfg: dict, cache: KVCache,
                logits_of=None) -> np.ndarray:
    """Greedy decoding of n_new tokens per sequence: step t decodes the
    previous token (first [B] at t = 0) and takes the greedy token of its
    logits.  logits_of(t, logits) may replace a step's logits (tests feed
    the device's own logits here so both sides take identical decisions).
    Returns int32 tokens [B, n_new]."""
    tok = np.asarray(first).reshape(-1).astype(np.int32)
    out = np.zeros((tok.size, n_new), dtype=np.int32)
    for t in range(n_new):
        lg = ar_decode_step(tok, W, cfg, cache)
        if logits_of is not None:
            lg = logits_of(t, lg)
        tok = greedy_token(lg)
        out[:, t] = tok
    return out


# ---------------------------------------------------------------- training forward
# Report-summary page, section 1: training replaces a random share of a
# sentence's tokens (from none to all) by junk and asks the model for the
# originals; section 3: the supervised stage does this at varying degrees
# and learns from the gap between prediction and original.  Plainest
# reading: multinomial corruption at a per-canvas rate (sampler.c,
# ora_corrupt), one denoiser forward of the corrupted canvas over the cached
# context with no self-conditioning input (there is no previous round), and
# the cross-entropy of each position's prediction at its clean token.

def xent_rows(logits: np.ndarray, target: np.ndarray) -> np.ndarray:
    """-log softmax(l)[x] per row of float64 logits [..., V] (the textbook
    log-sum-exp), target [...] int."""
    lg = np.asarray(logits, dtype=np.float64)
    m = lg.max(axis=-1, keepdims=True)
    lse = m[..., 0] + np.log(np.exp(lg - m).sum(axis=-1))
    lt = np.take_along_axis(lg, np.asarray(target)[..., None].astype(np.int64), axis=-1)[..., 0]
    return lse - lt


def train_forward(clean: np.ndarray, rate: np.ndarray, seed: int, step: int, W: dict, cfg: dict,
                  cache: KVCache):
    """Training-side forward of canvases clean [B, N] at corruption rates
    rate [B] over the cached context (not modified).  Returns (corrupted
    canvas int32 [B, N], float64 logits [B, N, V], float64 losses [B, N],
    their mean)."""
    from oracle import sampler as osampler
    clean = np.asarray(clean, dtype=np.int32)
    x = osampler.corrupt(seed, step, W["embed"].shape[0], np.asarray(rate, np.float32), clean)
    logits = denoise_step(x, W, cfg, cache)
    loss = xent_rows(logits, clean)
    return x, logits, loss, float(loss.mean())


def denoise_step(canvas: np.ndarray, W: dict, cfg: dict, cache: KVCache,
                 prev_logits: np.ndarray | None = None, top_k: int = 0) -> np.ndarray:
    """One denoiser forward over canvases [B, N] with bidirectional attention
    over [cached context ; canvas].  The cache is not modified.  Returns
    float64 logits [B, N, V]."""
    canvas = np.asarray(canvas)
    B, N = canvas.shape
    out = []
    for b in range(B):
        h = denoiser_input(canvas[b], W, None if prev_logits is None else prev_logits[b], top_k)
        for li, lw in enumerate(W["layers"]):
            h, _, _ = attn_half(h, lw, cfg, cache.k[li][b], cache.v[li][b], cache.length,
                                causal=False)
            h, _, _, _ = moe_half(h, lw, cfg)
        out.append(head(h, W, cfg))
    return np.stack(out)
