"""Block-autoregressive driver of the oracle (TEST INFRASTRUCTURE ONLY).

Report-summary page (animattoys.com), sections 1 and 4: a block starts as 256
uniformly random tokens and is refined for at most 48 rounds, each round
predicting every position, locking confident positions and re-randomising the
rest, until the entropy stop fires.  akiraxclaw.com blog, "memory, not
compute", and youleyou.com article, "Architecture basis": a finished block is
encoded into the KV cache and the next block is conditioned on it.

The block output is the most likely token sequence of the last round (the stop
rule is defined on it).  Committing re-encodes that block causally.  Each
canvas stops on its own; a stopped canvas is left as it is.

When the sampler truncates to each position's top_k logits (report-summary
page, section 9, names top-k truncation without defining it), the next
round's self-conditioning uses the same truncated distribution: the plainest
reading is that the model conditions on the distribution the sampler drew
from.
"""
from __future__ import annotations

import numpy as np

from . import model, sampler


def generate_block(W: dict, cfg: dict, cache: model.KVCache, params: dict, block_index: int,
                   B: int, selfcond: bool = True, logits_hook=None, round_hook=None):
    """Runs one block; returns (block tokens [B, N] int32, steps [B] int32).
    logits_hook(step, logits) may replace the float64 model logits (it must
    return a [B, N, V] array) -- tests use it to feed identical logits to
    two implementations.  round_hook(step, canvas, argmax, lock, stats, stop)
    observes the sampler's outputs after each round (it must not modify
    them)."""
    N, V = cfg["canvas"], cfg["vocab"]
    top_k = int(params.get("top_k", 0))
    canvas = sampler.canvas_init(params["seed"], block_index, B, N, V)
    argmax = np.zeros((B, N), dtype=np.int32)
    stop = np.zeros(B, dtype=np.int32)
    steps = np.zeros(B, dtype=np.int32)
    prev = None
    for t in range(params["max_steps"]):
        active = stop == 0
        if not active.any():
            break
        logits = model.denoise_step(canvas, W, cfg, cache, prev if selfcond else None,
                                    top_k=top_k if prev is not None else 0)
        if logits_hook is not None:
            logits = logits_hook(t, logits)
        logits32 = np.ascontiguousarray(logits, dtype=np.float32)
        lock, stats = sampler.sample_update(params, t, logits32, canvas, argmax, stop)
        if round_hook is not None:
            round_hook(t, canvas, argmax, lock, stats, stop)
        steps[active] = t + 1
        # a stopped canvas keeps its last logits for self-conditioning
        prev = logits32.astype(np.float64) if prev is None else np.where(
            active[:, None, None], logits32.astype(np.float64), prev)
    block = argmax.copy()
    model.encode(block, W, cfg, cache)
    return block, steps
