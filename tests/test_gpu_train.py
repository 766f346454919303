"""Training-side forward on the GPU through the C ABI: the multinomial
corruption and the binary32 cross-entropy bit-exact against the C oracle on
identical seeded inputs; the whole forward (corrupt, denoise, cross-entropy)
against the float64 oracle (fp32 1e-4, bf16 2e-2 on positions whose routes
are not within the GPU's precision of a tie) and bitwise equal to its own
composition of calls; a full-size layer (vocabulary 262144, prompt 2048) on
sampled positions."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic
from oracle import model as om
from oracle import sampler as osampler

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


# bf16 end to end on one layer, as the denoising-step tests: with more, a
# prompt token whose route the GPU's rounding flips changes its later
# layers' K/V, which every canvas position reads
@pytest.mark.parametrize("name,P,B,layers", [("tiny", 40, 2, 2), ("small_bf16", 120, 2, 1),
                                             ("f32_gqa", 33, 2, 2), ("small_fp8", 120, 1, 1)])
def test_train_forward_matches_oracle(name, P, B, layers):
    print(f"train forward {name} P={P} B={B} layers={layers}", flush=True)
    cfg, W, m = setup(name, P, batch=B, n_layers=layers)
    N, V = cfg["canvas"], cfg["vocab"]
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
    W64 = synthetic.to_float64(W)
    cache = om.KVCache(cfg, B)
    om.encode(prompt, W64, cfg, cache)
    xr, lr, ref_loss, ref_mean = om.train_forward(clean, rate, 31, 4, W64, cfg, cache)
    assert np.array_equal(x.cpu().numpy(), xr)
    # positions whose route is ambiguous at the GPU's precision are not compared
    keep = np.ones((B, N), dtype=bool)
    for b in range(B):
        h = om.embed(xr[b], W64)
        for li, lw in enumerate(W64["layers"]):
            h, _, _ = om.attn_half(h, lw, cfg, cache.k[li][b], cache.v[li][b], P, causal=False)
            u = om.rmsnorm(h, lw["moe_norm"], cfg["rms_eps"])
            keep[b] &= ~route_ambiguous(u @ lw["w_router"].T, cfg["top_k"],
                                        route_gap(cfg, chained=True))
            h, _, _, _ = om.moe_half(h, lw, cfg)
    assert keep.mean() > 0.5
    tol = tol_for(cfg)
    got_l = logits.cpu().numpy()
    assert normwise(got_l[keep], lr[keep]) <= tol
    got_loss = loss.cpu().numpy()
    assert normwise(got_loss[keep], ref_loss[keep]) <= tol
    assert abs(float(mean.cpu().numpy()[0]) - ref_mean) <= tol * abs(ref_mean)
    # the GPU mean is the sequential binary32 mean of its own losses
    acc = np.float32(0.0)
    for v in got_loss.reshape(-1):
        acc = np.float32(acc + v)
    assert mean.cpu().numpy()[0] == np.float32(acc / np.float32(B * N))


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


def test_train_forward_full_layer_sampled_rows():
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
    got_rows = logits[0].cpu().numpy()
    del m, logits
    torch.cuda.empty_cache()
    # the GPU's cross-entropy of its own logits, bit-exact, on sampled rows
    rows = np.arange(0, N, 16)
    ref_ce, _ = osampler.xent(got_rows[rows], clean[0, rows])
    assert np.array_equal(got_loss[rows], ref_ce)
    print("oracle encode + step", flush=True)
    SAMPLE = 16
    lw = {k: np.asarray(v, dtype=np.float64) if k.endswith("norm") or k in ("wq", "wk", "wv", "wo")
          else v for k, v in W["layers"][0].items()}
    Wk = {"embed": W["embed"], "w_sc": W["w_sc"], "final_norm": W["final_norm"], "layers": [lw]}
    cache = om.KVCache(cfg, 1)
    om.encode(prompt, Wk, cfg, cache)
    h = om.embed(xg[0], Wk)
    h, _, _ = om.attn_half(h, lw, cfg, cache.k[0][0], cache.v[0][0], P, causal=False)
    u = om.rmsnorm(h, lw["moe_norm"], cfg["rms_eps"])
    amb = route_ambiguous(u @ np.asarray(lw["w_router"], np.float64).T, cfg["top_k"], 3e-2)
    h, _, _, _ = om.moe_half(h, lw, cfg)
    # sampled among the positions whose route is not within bf16 precision
    # of a tie
    ok = np.flatnonzero(~amb)
    keep = ok[np.linspace(0, ok.size - 1, SAMPLE).astype(int)]
    ref = om.xent_rows(om.head(h[keep], Wk, cfg), clean[0, keep])
    err = normwise(got_loss[keep], ref)
    print(f"full-layer loss normwise error {err:.3e} over {keep.size} rows", flush=True)
    assert err <= TOL_BF16
