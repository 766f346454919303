"""Attention at the long-context and batched shapes against the float64
oracle on synthetic caches: the full-size attention block (d 2048, 16 query /
4 KV heads x 128, bf16) of a 256-token canvas over a 32768-token context
(33024 keys, the long-generation workload; also causal, as a block commit at
that length runs it), and eight canvases over 8192-token contexts each (8448
keys, the batched workload).  Every query of every sequence is compared
(output of the attention block and the canvas K/V it writes), so a key-range
split that drops, repeats or misweights a range would show."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic

import chain
from helpers import DEV, TOL_BF16, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


@pytest.mark.parametrize("B,P,causal", [(1, 32768, False), (1, 32768, True), (8, 8192, False)])
def test_attention_long_context(B, P, causal):
    print(f"attention over a synthetic cache: batch {B}, context {P}, causal {causal}", flush=True)
    # the attention block's shapes; a small vocabulary and expert set (unused here)
    cfg = synthetic.model_config("layer", vocab=1024, n_experts=8, top_k=2)
    N, d = cfg["canvas"], cfg["d_model"]
    W = synthetic.make_weights(cfg, seed=21, random_norms=True)
    m = binding.Model(cfg, W, batch=B, capacity=P + N)
    K, V = m.kv_tensors()
    g = torch.Generator(device=DEV)
    g.manual_seed(22)
    K[0, :, :, :P] = (2.0 * torch.randn(K[0, :, :, :P].shape, generator=g, device=DEV)).to(K.dtype)
    V[0, :, :, :P] = torch.randn(V[0, :, :, :P].shape, generator=g, device=DEV).to(V.dtype)
    m.set_kv_length(P)
    h = to_dev(np.random.default_rng(23).standard_normal((B * N, d)).astype(np.float32))
    torch.cuda.synchronize()
    chain.check_attention(m, cfg, chain.layer64(W["layers"][0]), 0, h, N, causal, TOL_BF16,
                          label=f"B={B} P={P}")
