"""Training-side forward on the GPU through the C ABI: the multinomial
corruption and the binary32 cross-entropy bit-exact against the C oracle on
identical seeded inputs; the whole forward (corrupt, denoise, cross-entropy)
against the float64 oracle stage by stage on the GPU's own inputs (fp32
1e-4, bf16 2e-2, every position) and bitwise equal to its own composition of
calls; a full-size layer (vocabulary 262144, prompt 2048) at every
position."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic
from oracle import model as om
from oracle import sampler as osampler

import chain
from helpers import DEV, TOL_BF16, normwise, route_ambiguous, to_dev, tol_for

pytestmark = pytest.mark.gpu

from test_gpu_model import route_gap, setup  # noqa: E402


@pytest.mark.parametrize("B,N,V,seed,step", [(3, 256, 262144, 5, 0), (4, 100, 1000, 77, 9),
                                             (1, 1, 2, 0, 0), (2, 256, 4096, 2**63 + 5, 47)])
def test_corrupt_bit_exact(B, N, V, seed, step):
    print(f"corrupt B={B} N={N} V={V}", flush=True)
    clean = synthetic.make_tokens(V, (B, N), seed=3)
    rate = np.linspace(0.0, 1.0, B).astype(np.float32)
    if B == 4:
        rate = np.array([0.0, 0.05, 0.5, 1.0], np.float32)
    out = torch.full((B, N), -1, dtype=torch.int32, device=DEV)
    binding.corrupt(seed, step, V, to_dev(rate), to_dev(clean), out)
    torch.cuda.synchronize()
    ref = osampler.corrupt(seed, step, V, rate, clean)
    assert np.array_equal(out.cpu().numpy(), ref)


XENT_CASES = [(7, 262144, "normal"), (5, 65536 + 77, "normal"), (4, 1001, "flat"),
              (3, 4, "normal"), (6, 4096, "sharp"), (2, 131072, "ties")]


@pytest.mark.parametrize("R,V,kind", XENT_CASES)
def test_xent_bit_exact(R, V, kind):
    print(f"xent R={R} V={V} {kind}", flush=True)
    lg = synthetic.make_logits((R, V), seed=R * 31 + V, sigma=2.0)
    if kind == "flat":
        lg[:] = 0.25
    elif kind == "sharp":
        lg[:, 7] = 70.0
    elif kind == "ties":
        lg[:, 10] = lg[:, 20000] = 9.0
    tgt = synthetic.make_tokens(V, (R,), seed=R)
    tgt[0] = 0
    tgt[-1] = V - 1
    loss = torch.empty(R, dtype=torch.float32, device=DEV)
    mean = torch.empty(1, dtype=torch.float32, device=DEV)
    binding.xent(to_dev(lg), to_dev(tgt), loss, mean)
    torch.cuda.synchronize()
    ref, ref_mean = osampler.xent(lg, tgt)
    assert np.array_equal(loss.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert mean.cpu().numpy()[0].view(np.uint32) == np.float32(ref_mean).view(np.uint32)


def test_xent_target_outside_vocab_is_nan():
    lg = synthetic.make_logits((3, 500), seed=1)
    tgt = np.array([5, -1, 500], np.int32)
    loss = torch.empty(3, dtype=torch.float32, device=DEV)
    binding.xent(to_dev(lg), to_dev(tgt), loss)
    torch.cuda.synchronize()
    got = loss.cpu().numpy()
    ref, _ = osampler.xent(lg[:1], tgt[:1])
    assert got[0] == ref[0]
    assert np.isnan(got[1]) and np.isnan(got[2])


@pytest.mark.parametrize("name,P,B,layers", [("tiny", 40, 2, 2), ("small_bf16", 120, 2, 2),
                                             ("f32_gqa", 33, 2, 2), ("small_fp8", 120, 1, 2),
                                             ("small_mxfp4", 120, 1, 2)])
def test_train_forward_matches_oracle(name, P, B, layers):
    """The corrupted canvas bit-exact against the oracle; the cross-entropy
    bit-exact against the oracle's on the GPU's own logits, every row; the
    mean the sequential binary32 mean; the logits as a chain of the
    forward's stages, each against the oracle on the GPU's own input (the
    MoE with the GPU's route set), every position, equal to the forward's
    bit for bit; fp32 models also end to end against the oracle's own
    forward (positions within 1e-4 of a router tie, at most 1 %, skipped)."""
    print(f"train forward {name} P={P} B={B} layers={layers}", flush=True)
    cfg, W, m = setup(name, P, batch=B, n_layers=layers)
    N, V, d = cfg["canvas"], cfg["vocab"], cfg["d_model"]
    prompt = synthetic.make_tokens(V, (B, P), seed=21)
    clean = synthetic.make_tokens(V, (B, N), seed=22)
    rate = np.linspace(0.2, 0.9, B).astype(np.float32)
    m.encode_prompt(to_dev(prompt))
    x = torch.empty((B, N), dtype=torch.int32, device=DEV)
    logits = torch.empty((B, N, V), dtype=torch.float32, device=DEV)
    loss = torch.empty((B, N), dtype=torch.float32, device=DEV)
    mean = torch.empty(1, dtype=torch.float32, device=DEV)
    m.train_forward(to_dev(clean), to_dev(rate), 31, 4, x, logits, loss, mean)
    torch.cuda.synchronize()
    assert m.kv_length == P
    xg = x.cpu().numpy()
    assert np.array_equal(xg, osampler.corrupt(31, 4, V, rate, clean))
    got_loss = loss.cpu().numpy()
    ref_ce, _ = osampler.xent(logits.cpu().numpy().reshape(B * N, V), clean.reshape(-1))
    assert np.array_equal(got_loss.reshape(-1).view(np.uint32), ref_ce.view(np.uint32))
    acc = np.float32(0.0)
    for v in got_loss.reshape(-1):
        acc = np.float32(acc + v)
    assert mean.cpu().numpy()[0] == np.float32(acc / np.float32(B * N))
    # the forward's stages on the corrupted canvas
    tol = tol_for(cfg)
    W64 = synthetic.to_float64(W)
    h = torch.empty((B * N, d), dtype=torch.float32, device=DEV)
    m.stage_input(x, h)
    for l, lw in enumerate(W["layers"]):
        lw = chain.layer64(lw)
        chain.check_attention(m, cfg, lw, l, h, N, False, tol, label=f"train {name}")
        chain.check_moe(m, cfg, lw, l, h, tol, label=f"train {name}")
    lc = chain.check_head(m, cfg, W64, h, tol, label=f"train {name}")
    assert torch.equal(lc.view(B, N, V), logits)
    if cfg["dtype"] != "f32":
        return
    cache = om.KVCache(cfg, B)
    om.encode(prompt, W64, cfg, cache)
    xr, lr, ref_loss, ref_mean = om.train_forward(clean, rate, 31, 4, W64, cfg, cache)
    keep = np.ones((B, N), dtype=bool)
    for b in range(B):
        hh = om.embed(xr[b], W64)
        for li, lw in enumerate(W64["layers"]):
            hh, _, _ = om.attn_half(hh, lw, cfg, cache.k[li][b], cache.v[li][b], P, causal=False)
            u = om.rmsnorm(hh, lw["moe_norm"], cfg["rms_eps"])
            keep[b] &= ~route_ambiguous(u @ lw["w_router"].T, cfg["top_k"], route_gap(cfg))
            hh, _, _, _ = om.moe_half(hh, lw, cfg)
    assert keep.mean() >= 0.99
    assert normwise(logits.cpu().numpy()[keep], lr[keep]) <= tol
    assert normwise(got_loss[keep], ref_loss[keep]) <= tol


def test_train_forward_equals_composition():
    cfg, W, m = setup("small_bf16", 60, batch=2)
    N, V = cfg["canvas"], cfg["vocab"]
    m.encode_prompt(to_dev(synthetic.make_tokens(V, (2, 60), seed=1)))
    clean = to_dev(synthetic.make_tokens(V, (2, N), seed=2))
    rate = to_dev(np.array([0.0, 0.6], np.float32))
    x = torch.empty((2, N), dtype=torch.int32, device=DEV)
    lg = torch.empty((2, N, V), dtype=torch.float32, device=DEV)
    loss = torch.empty((2, N), dtype=torch.float32, device=DEV)
    m.train_forward(clean, rate, 8, 1, x, lg, loss)
    x2 = torch.empty_like(x)
    binding.corrupt(8, 1, V, rate, clean, x2)
    lg2 = torch.empty_like(lg)
    m.denoise_step(x2, lg2)
    loss2 = torch.empty_like(loss)
    binding.xent(lg2.view(-1, V), clean.view(-1), loss2.view(-1))
    torch.cuda.synchronize()
    assert torch.equal(x, x2) and torch.equal(x[0], clean[0])
    assert torch.equal(lg, lg2)
    assert torch.equal(loss, loss2)


def test_train_forward_full_layer():
    cfg = synthetic.model_config("layer")
    P, N, V = synthetic.SHAPES["layer"]["prompt"], cfg["canvas"], cfg["vocab"]
    print("generating full-size layer weights", flush=True)
    W = synthetic.make_weights(cfg, seed=0)
    prompt = synthetic.make_tokens(V, (1, P), seed=1)
    clean = synthetic.make_tokens(V, (1, N), seed=2)
    rate = np.array([0.5], np.float32)
    m = binding.Model(cfg, W, batch=1, capacity=P + N)
    m.encode_prompt(to_dev(prompt))
    x = torch.empty((1, N), dtype=torch.int32, device=DEV)
    logits = torch.empty((1, N, V), dtype=torch.float32, device=DEV)
    loss = torch.empty((1, N), dtype=torch.float32, device=DEV)
    mean = torch.empty(1, dtype=torch.float32, device=DEV)
    m.train_forward(to_dev(clean), to_dev(rate), 3, 0, x, logits, loss, mean)
    torch.cuda.synchronize()
    xg = x.cpu().numpy()
    assert np.array_equal(xg, osampler.corrupt(3, 0, V, rate, clean))
    got_loss = loss.cpu().numpy()[0]
    # the GPU's cross-entropy of its own logits, bit-exact, at every row
    ref_ce, _ = osampler.xent(logits[0].cpu().numpy(), clean[0])
    assert np.array_equal(got_loss, ref_ce)
    # the forward as a chain of its stages on the corrupted canvas, each
    # against the oracle on the GPU's own input (the MoE with the GPU's
    # route set), every position; the chain equals the forward bit for bit
    print("stage chain against the oracle", flush=True)
    lw = chain.layer64(W["layers"][0])
    Wk = {"embed": W["embed"], "w_sc": W["w_sc"], "final_norm": W["final_norm"], "layers": [lw]}
    h = torch.empty((N, cfg["d_model"]), dtype=torch.float32, device=DEV)
    m.stage_input(x, h)
    torch.cuda.synchronize()
    assert normwise(h.cpu().numpy(), om.embed(xg[0], Wk)) == 0.0
    chain.check_attention(m, cfg, lw, 0, h, N, False, TOL_BF16, label="train")
    chain.check_moe(m, cfg, lw, 0, h, TOL_BF16, label="train")
    lc = chain.check_head(m, cfg, Wk, h, TOL_BF16, label="train")
    assert torch.equal(lc.view(1, N, V), logits)
    # the oracle's loss on the chain's final hidden state, every position
    ref = om.xent_rows(om.head(h.cpu().numpy().astype(np.float64), Wk, cfg), clean[0])
    err = normwise(got_loss, ref)
    print(f"full-layer loss normwise error {err:.3e} over {N} rows", flush=True)
    assert err <= TOL_BF16
