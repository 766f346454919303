"""dg_sample_update_static (the sampler update for callers that cannot allocate:
its scratch is a static device array inside the library) against
dg_sample_update with a caller workspace, through the C ABI: two calls in a
row, the second with a smaller input (the static array keeps the first
call's contents), bit for bit on every output, with a stopped canvas, locks
on part of the rows, both lock rules and top-k truncation.  A request above
the array's limit is refused before anything is launched."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic

from helpers import DEV

pytestmark = pytest.mark.gpu

# (batch, canvas, vocab, lock rule, top_k): the second call is smaller
CALLS = [(4, 256, 4096, binding.LOCK_CUMENT, 0), (1, 100, 1000, binding.LOCK_MAXPROB, 8)]


def inputs(B, N, V, seed):
    rng = np.random.default_rng(seed)
    # per-row sharpness from flat to nearly certain, so some rows lock
    sigma = np.exp(rng.uniform(np.log(0.5), np.log(40.0), size=(B, N, 1)))
    logits = (rng.standard_normal((B, N, V)) * sigma).astype(np.float32)
    canvas = rng.integers(0, V, size=(B, N)).astype(np.int32)
    argmax = rng.integers(0, V, size=(B, N)).astype(np.int32)
    stop = np.zeros(B, np.int32)
    if B > 1:
        stop[1] = 1          # a stopped canvas is left untouched
    return logits, canvas, argmax, stop


def run(static, params, step, logits, canvas, argmax, stop):
    B, N, V = logits.shape
    t = lambda a: torch.from_numpy(a.copy()).to(DEV)   # noqa: E731
    lg, cv, am, sp = t(logits), t(canvas), t(argmax), t(stop)
    lock = torch.full((B, N), 7, dtype=torch.uint8, device=DEV)
    stats = torch.full((B, N, 4), -1.0, dtype=torch.float32, device=DEV)
    if static:
        binding.sample_update_static(params, step, lg, cv, am, lock, stats, sp)
    else:
        ws = binding.sampler_workspace(B, N)
        binding.sample_update(params, step, lg, cv, am, lock, stats, sp, ws)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (cv, am, lock, stats, sp)]


def test_static_sampler_equals_workspace_sampler():
    for i, (B, N, V, rule, top_k) in enumerate(CALLS):
        print(f"call {i}: batch {B} canvas {N} vocab {V} rule {rule} top_k {top_k}", flush=True)
        logits, canvas, argmax, stop = inputs(B, N, V, 60 + i)
        params = synthetic.default_sampler_params(max_steps=8, seed=11 + i, lock_rule=rule,
                                                  lock_theta=0.9 if rule == binding.LOCK_MAXPROB
                                                  else 0.1, top_k=top_k)
        ref = run(False, params, 3, logits, canvas, argmax, stop)
        got = run(True, params, 3, logits, canvas, argmax, stop)
        for name, a, b in zip(("canvas", "argmax", "lock", "stats", "stop"), got, ref):
            assert a.dtype == b.dtype and a.shape == b.shape
            assert (a.view(np.uint8) == b.view(np.uint8)).all(), f"call {i}: {name} differs"
        assert ref[2].any() and not ref[2][stop == 0].all(), "some rows should lock"


def test_static_sampler_refuses_above_its_limit():
    B, N, V = 65, 1024, 8          # 66560 rows > 65536
    logits = torch.zeros((B, N, V), dtype=torch.float32, device=DEV)
    canvas = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    argmax = torch.zeros_like(canvas)
    lock = torch.zeros((B, N), dtype=torch.uint8, device=DEV)
    stats = torch.zeros((B, N, 4), dtype=torch.float32, device=DEV)
    stop = torch.zeros(B, dtype=torch.int32, device=DEV)
    with pytest.raises(binding.DGError) as e:
        binding.sample_update_static(synthetic.default_sampler_params(), 0, logits, canvas, argmax,
                                     lock, stats, stop)
    assert e.value.status == 4
