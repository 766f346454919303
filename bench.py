#!/usr/bin/env python3
"""Benchmark of the block text-diffusion denoising path on one MI355X.

One benchmark step = one block of block-autoregressive generation through
the whole hot path (dg_generate_block): canvas initialisation, up to 48
rounds of [self-conditioning + embedding, the denoiser layer stack with
bidirectional attention over the cached prompt, top-8-of-128 MoE, tied
vocabulary head, sampler with lock / renoise / entropy stop], then the
causal commit of the block into the KV cache.  The cache is rewound to the
prompt after each block so every step does identical work.

Prints one JSON line.  value = canvas tokens per second (finished block
tokens / wall time); ms_per_step = one block.  With random-init weights the
entropy stop never fires, so each block runs the full 48 rounds.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
                  [--config layer|layer_fp8|layer_mxfp4|stack|batched|long] [--layers L] [--top-k K]
  python bench.py --mode train [--rate r] [--config ...]
      the training-side forward: value = canvas tokens/s through corruption,
      the denoiser forward and the cross-entropy at the clean tokens
  python bench.py --mode ar [--ar-tokens n] [--ar-batch B] [--config ...]
      the retained autoregressive mode: value = decoded tokens/s (greedy
      decoding of n tokens per sequence after the prompt, B sequences)
  python bench.py --mode moe [--config ...]
      the mixture-of-experts half alone: value = HBM GB/s of the two expert
      products (dg_stage_moe of the configuration's canvases)
  python bench.py --mode attn [--config ...]
      the attention block alone (dg_stage_attention) of the configuration's
      canvases over a synthetic cache of its context length: value =
      attention TFLOP/s (the kernel and its split merge, library timer)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # FLOP per byte
# fp32 vector ALU without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# binary32 operations per second (an fma counts as one operation here)
ALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
ALU_RIDGE = ALU_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # operations per byte
# binary32 operations per logit of the sampler's row pass, from its
# definition: chunk max 1, z = l - m 1, E(z) 14, three sums and e*z 4,
# z*invT 1, E(z*invT) 14, plus 2 when it also writes the self-conditioning
# weight (e*f and the bf16 conversion)
SAMPLER_OPS = 36


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="layer",
                    choices=["layer", "layer_fp8", "layer_mxfp4", "stack", "batched", "long"])
    ap.add_argument("--layers", type=int, default=None,
                    help="override the configuration's layer count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true",
                    help="layer workload: skip the 30-layer stack measurement that the default "
                         "run adds under the key \"stack\"")
    ap.add_argument("--stack-steps", type=int, default=2,
                    help="timed blocks of the 30-layer stack measurement")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the microbenchmark peaks (HBM read and copy, bf16 matrix "
                         "product) reported beside the published ones")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the measurement, two 1 GiB device copies (counter calibration)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--top-k", type=int, default=0,
                    help="sampler top-k truncation (0: the full distribution)")
    ap.add_argument("--mode", default="diffusion", choices=["diffusion", "ar", "train", "attn", "moe"],
                    help="ar: the retained autoregressive mode (greedy decoding); one step "
                         "= --ar-tokens tokens per sequence after the prompt.  train: the "
                         "training-side forward; one step = corruption + denoiser forward + "
                         "cross-entropy of every canvas")
    ap.add_argument("--rate", type=float, default=0.5,
                    help="train: corruption rate of every canvas")
    ap.add_argument("--router-skew", action="store_true",
                    help="--mode moe: inject the router logits N(0,1) + 0.5 on 13 hot experts "
                         "(the batched workload's expert skew) instead of computing them from "
                         "random router weights; reports the measured max/mean expert load")
    ap.add_argument("--ar-tokens", type=int, default=64)
    ap.add_argument("--ar-batch", type=int, default=1)
    return ap.parse_args()


def device_weights(cfg, seed, torch):
    """Random-init weights N(0, 0.02^2) drawn on the GPU (torch's generator),
    rounded once to bf16; RMSNorm scales are ones."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    d, V = cfg["d_model"], cfg["vocab"]
    Hq, Hkv, dh, E, F = (cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["n_experts"],
                         cfg["d_ff"])

    def draw(*shape):
        return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * 0.02).to(dt)

    def ones():
        return torch.ones(d, device="cuda", dtype=torch.float32)

    W = {"embed": draw(V, d), "w_sc": draw(d, d), "final_norm": ones(), "layers": []}
    for _ in range(cfg["n_layers"]):
        lw = {"attn_norm": ones(), "wq": draw(Hq * dh, d), "wk": draw(Hkv * dh, d),
              "wv": draw(Hkv * dh, d), "wo": draw(d, Hq * dh), "moe_norm": ones(),
              "w_router": draw(E, d), "w_gate": draw(E, F, d), "w_up": draw(E, F, d),
              "w_down": draw(E, d, F)}
        if cfg.get("expert_dtype") == "fp8":
            # 8-bit experts: the same draws, quantised on the GPU by the
            # library (E4M3 codes, one scale per weight row)
            from discrete_text_diffusion_denoise_amd import binding
            for k, sk in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down")):
                w = lw[k]
                q = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
                sc = torch.empty(w.shape[:-1], dtype=torch.float32, device="cuda")
                binding.quantize_fp8(w, q, sc)
                lw[k], lw[sk] = q, sc
            torch.cuda.synchronize()
        if cfg.get("expert_dtype") == "mxfp4":
            # MXFP4 experts: the same draws, quantised on the GPU by the
            # library (packed E2M1 codes, an E8M0 scale per 32 weights)
            from discrete_text_diffusion_denoise_amd import binding
            for k, xk in (("w_gate", "x_gate"), ("w_up", "x_up"), ("w_down", "x_down")):
                w = lw[k]
                q = torch.empty(w.shape[:-1] + (w.shape[-1] // 2,), dtype=torch.uint8, device="cuda")
                sc = torch.empty(w.numel() // 32, dtype=torch.uint8, device="cuda")
                binding.quantize_mxfp4(w, q, sc)
                lw[k], lw[xk] = q, sc
            torch.cuda.synchronize()
        W["layers"].append(lw)
    return W


def kernel_work(name, cfg, B, P, sc_splits):
    """Algorithmic (flops, bytes) of one launch of a timed kernel: every
    weight read once, activations read/written once.  cfg["canvas"] is the
    number of new tokens per sequence (1 in the autoregressive mode)."""
    es = 2 if cfg["dtype"] == "bf16" else 4
    # expert weight bytes per element (8-bit experts also read one fp32
    # scale per weight row)
    fp8 = cfg.get("expert_dtype") == "fp8"
    fp4 = cfg.get("expert_dtype") == "mxfp4"
    # MXFP4: half a byte per weight plus one scale byte per 32
    ew = 1 if fp8 else (0.5 + 1.0 / 32 if fp4 else es)
    N, V, d = cfg["canvas"], cfg["vocab"], cfg["d_model"]
    Hq, Hkv, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    E, k, F = cfg["n_experts"], cfg["top_k"], cfg["d_ff"]
    T = B * N
    # experts that receive at least one of the T*k assignments: measured from
    # the routes when the caller has them, else the uniform-routing estimate
    hit = cfg.get("experts_hit") or E * (1.0 - (1.0 - k / E) ** T)
    if name == "head_gemm":
        return 2.0 * T * V * d, V * d * es + T * d * es + T * V * 4.0
    if name == "selfcond_gemm":
        # bf16 models read the softmax probabilities in bf16 (written by a pre-pass)
        return 2.0 * T * d * V, T * V * es + d * V * es + sc_splits * T * d * 4.0
    # quantised experts take MXFP8 activations: a code byte per element and a
    # scale byte per 32
    ea = 1.0 + 1.0 / 32 if (fp8 or fp4) else es
    if name == "moe_gateup":
        return (2.0 * T * k * 2 * F * d,
                hit * 2 * F * (d * ew + (4 if fp8 else 0)) + T * d * ea + T * k * F * ea)
    if name == "moe_down":
        return (2.0 * T * k * F * d,
                hit * d * (F * ew + (4 if fp8 else 0)) + T * k * F * ea + T * k * d * 4.0)
    if name == "attention":
        L = P + N
        return (4.0 * T * L * Hq * dh,
                T * Hq * dh * es + B * L * Hkv * dh * 2 * es + T * Hq * dh * es)
    if name == "sampler":
        if cfg.get("sampler_alu"):
            # ALU work of the full-distribution row pass (see SAMPLER_OPS)
            ops = T * V * (SAMPLER_OPS + (2 if cfg.get("sampler_probs") else 0))
            nbytes = T * V * 4.0 + T * 16.0 + (T * V * 2.0 if cfg.get("sampler_probs") else 0.0)
            return ops, nbytes
        if cfg.get("sampler_top_k"):
            # slab maxima, then about K candidate slabs of 64 logits per row
            K = cfg["sampler_top_k"]
            return 0.0, T * (V / 64) * 4.0 + T * K * 64 * 4.0 + T * 16.0
        return 0.0, T * V * 4.0 + T * 16.0
    raise KeyError(name)


def roofline(name, ms, cfg, B, P, sc_splits):
    flops, nbytes = kernel_work(name, cfg, B, P, sc_splits)
    if name == "sampler" and cfg.get("sampler_alu") and flops / nbytes >= ALU_RIDGE:
        ach = flops / (ms * 1e-3) / 1e12
        return {"bound": "alu", "achieved": round(ach, 2), "peak": round(ALU_PEAK_TOPS, 1),
                "unit": "Top/s", "frac": round(ach / ALU_PEAK_TOPS, 4), "traffic": None,
                "kernel": name, "op_per_launch": flops, "bytes_per_launch": nbytes,
                "avg_launch_ms": round(ms, 5)}
    ai = flops / nbytes if nbytes else 0.0
    s = ms * 1e-3
    if flops and ai >= RIDGE:
        ach = flops / s / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": name, "flop_per_launch": flops, "bytes_per_launch": nbytes,
                "avg_launch_ms": round(ms, 5)}
    ach = nbytes / s / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": name,
            "flop_per_launch": flops, "bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 5)}


# kernel timer -> the source file its kernel is built from
KERNEL_SOURCE = {"head_gemm": "gemm_dma.hip", "selfcond_gemm": "gemm_dma.hip",
                 "moe_gateup": "moe.hip", "moe_down": "moe.hip", "attention": "attention.hip",
                 "sampler": "sampler.hip"}


def measured_traffic(name, config, source=None):
    """HBM bytes per launch of `name` from the committed counter summary
    profiles/traffic_<name>_<config>.txt (FETCH_SIZE and WRITE_SIZE runs,
    each scaled by the same counter on a 1 GiB copy), or None when there is
    no summary or the kernel's source (`source`, else the timer's usual
    file, and the header the summary names) has changed since it was
    taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{name}_{config}.txt")
    src = os.path.join(ROOT, "discrete_text_diffusion_denoise_amd", "csrc",
                       source or KERNEL_SOURCE.get(name, ""))
    if not os.path.exists(path) or not os.path.isfile(src):
        return None, None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    stale = vals.get("source_sha256") != digest or "traffic_bytes" not in vals
    if "header" in vals:
        # a header the kernel's code comes from (the LDS ring helpers)
        hdr = os.path.join(ROOT, vals["header"])
        stale = stale or not os.path.isfile(hdr) or \
            hashlib.sha256(open(hdr, "rb").read()).hexdigest() != vals.get("header_sha256")
    if stale:
        return None, os.path.relpath(path, ROOT) + " (stale: kernel source changed)"
    return float(vals["traffic_bytes"]), os.path.relpath(path, ROOT)


def copy_probe(torch):
    """Two 1 GiB device-to-device copies: the calibration of the HBM byte
    counters (a copy's bytes are known)."""
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def measured_peaks(torch):
    """Microbenchmark peaks of this GPU, reported beside the published ones
    (8 TB/s, 2.5 PFLOP/s bf16 dense): the library's probe kernels
    (dg_measure_peaks: a read-only stream over 4 GiB, independent bf16
    MFMAs at eight waves a SIMD), plus a 2 GiB device-to-device copy (read +
    write bytes) and a bf16 8192^3 torch.matmul (the vendor GEMM library) for
    context.  Calibration runs outside the timed region, not steps of the
    path."""
    from discrete_text_diffusion_denoise_amd import binding
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps * 1e-3

    buf = torch.empty(1 << 30, dtype=torch.float32, device="cuda")
    read_gbs, mfma_tf = binding.measure_peaks(buf)
    y = torch.empty(1 << 29, dtype=torch.float32, device="cuda")
    t_copy = timed(lambda: y.copy_(buf[: 1 << 29]), 10)
    del buf, y
    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    t_mm = timed(lambda: torch.matmul(a, b, out=c), 10)
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": round(read_gbs, 1),
            "bf16_mfma_tflops": round(mfma_tf, 1),
            "hbm_copy_gbs": round(2.0 * 4.0 * (1 << 29) / t_copy / 1e9, 1),
            "torch_matmul_bf16_tflops": round(2.0 * n ** 3 / t_mm / 1e12, 1),
            "method": "dg_measure_peaks (read-only stream over 4 GiB; independent "
                      "v_mfma_f32_16x16x32_bf16, eight waves a SIMD); 2 GiB device copy "
                      "(read + write bytes); bf16 8192^3 torch.matmul; outside the timed "
                      "region"}


def cpu_baseline(cfg, W, prompt, canvas, params, torch):
    """The CPU oracle (float64 numpy model + C sampler), timed on this host on
    a bounded sample: one self-conditioned denoising step and one sampler
    update over the full canvas, plus the commit encode; a block is 48 such
    rounds + a commit, so tokens/s = B*N / (48 * (step + sampler) + commit)."""
    import numpy as np
    from oracle import model as om
    from oracle import sampler as osampler
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    host = {"embed": W["embed"].float().cpu().numpy(), "w_sc": W["w_sc"].float().cpu().numpy(),
            "final_norm": W["final_norm"].cpu().numpy().astype(np.float64), "layers": []}
    for lw in W["layers"]:
        hl = {k: v.float().cpu().numpy() for k, v in lw.items()
              if not k.startswith("s_") and not k.startswith("x_")}
        if cfg.get("expert_dtype") == "mxfp4":
            # the oracle's experts are the dequantised MXFP4 weights, read
            # back out of the library's tiled layout (16-row tiles of
            # 128-column steps; chunk 16 g + r = row r's 32-column block g)
            from oracle import quant as oq
            for k, xk in (("w_gate", "x_gate"), ("w_up", "x_up"), ("w_down", "x_down")):
                q = lw[k].cpu().numpy()
                K = 2 * q.shape[-1]
                R = q.size // q.shape[-1]
                S = K // 128
                packed = q.reshape(R // 16, S, 4, 16, 16).transpose(0, 3, 1, 2, 4).reshape(R, K // 2)
                sc = lw[xk].cpu().numpy().reshape(R // 16, S, 4, 16).transpose(0, 3, 1, 2).reshape(
                    R, K // 32)
                hl[k] = oq.mx_dequantize_rows(oq.mx_unpack(packed), sc).reshape(q.shape[:-1] + (K,))
        if cfg.get("expert_dtype") == "fp8":
            # the oracle's experts are the dequantised codes, read back out of
            # the tiled layout (two 64-column halves a step, chunk 16 g + r)
            from oracle import quant as oq
            for k, sk in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down")):
                q = lw[k].cpu().numpy()
                K = q.shape[-1]
                R = q.size // K
                rows = q.reshape(R // 16, K // 128, 2, 4, 16, 16).transpose(0, 4, 1, 2, 3, 5).reshape(R, K)
                sc = lw[sk].cpu().numpy()
                hl[k] = oq.dequantize_rows(rows, sc.reshape(-1)).reshape(q.shape)
        host["layers"].append(hl)
    B, N, V = canvas.shape[0], cfg["canvas"], cfg["vocab"]
    P = prompt.shape[1]
    cache = om.KVCache(cfg, B)
    om.encode(prompt, host, cfg, cache)                 # prompt encode: not timed
    rng = np.random.default_rng(0)
    prev = (rng.standard_normal((B, N, V), dtype=np.float32) * 2.0)
    t0 = time.perf_counter()
    logits = om.denoise_step(canvas, host, cfg, cache, prev)
    t1 = time.perf_counter()
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    cv = canvas.astype(np.int32).copy()
    am = np.zeros((B, N), np.int32)
    stop = np.zeros(B, np.int32)
    osampler.sample_update(params, 0, lg, cv, am, stop)
    t2 = time.perf_counter()
    om.encode(cv, host, cfg, cache)                     # commit of one block
    t3 = time.perf_counter()
    block_s = 48 * ((t1 - t0) + (t2 - t1)) + (t3 - t2)
    return {"value": round(B * N / block_s, 4), "unit": "canvas tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"one self-conditioned denoise step ({(t1 - t0):.2f} s, float64 numpy, "
                       f"{threads} BLAS threads) + one sampler update over {B}x{N} rows of "
                       f"{V} logits ({(t2 - t1):.2f} s, C, 1 thread) + one {N}-token commit "
                       f"({(t3 - t2):.2f} s) at prompt {P}; block = 48 rounds + commit, "
                       f"extrapolated"),
            "step_s": round(t1 - t0, 3), "sampler_s": round(t2 - t1, 3),
            "commit_s": round(t3 - t2, 3)}


def cpu_baseline_ar(cfg, W, prompt, B):
    """The CPU oracle's autoregressive decode step (float64 numpy), timed on
    this host: the prompt encode is not timed, then one decode step of the B
    sequences; tokens/s = B / step time (the oracle runs the sequences one
    after another, so one sequence gives the rate of any batch)."""
    import numpy as np
    from oracle import model as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    host = {"embed": W["embed"].float().cpu().numpy(), "w_sc": W["w_sc"].float().cpu().numpy(),
            "final_norm": W["final_norm"].cpu().numpy().astype(np.float64), "layers": []}
    for lw in W["layers"]:
        host["layers"].append({k: v.float().cpu().numpy() for k, v in lw.items()
                               if not k.startswith("s_")})
    P = prompt.shape[1]
    cache = om.KVCache(cfg, B)
    om.encode(prompt[:, :P - 1], host, cfg, cache)
    t0 = time.perf_counter()
    om.ar_decode_step(prompt[:, P - 1], host, cfg, cache)
    t1 = time.perf_counter()
    return {"value": round(B / (t1 - t0), 4), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"one decode step of {B} sequence(s) after a {P - 1}-token prompt "
                       f"({(t1 - t0):.2f} s, float64 numpy, {threads} BLAS threads)")}


def bench_ar(args):
    """The retained autoregressive mode: one step = greedy decoding of
    --ar-tokens tokens for each of --ar-batch sequences after the prompt
    (dg_ar_generate); the cache is rewound to the prompt after each step."""
    import numpy as np
    import torch

    from discrete_text_diffusion_denoise_amd import binding, synthetic

    shape = synthetic.SHAPES[args.config]
    over = {"n_layers": args.layers} if args.layers else {}
    cfg = synthetic.model_config(args.config, **over)
    if cfg.get("expert_dtype"):
        raise SystemExit("--mode ar runs the bf16 configurations")
    B, P, V, n_new = args.ar_batch, shape["prompt"], cfg["vocab"], args.ar_tokens
    torch.cuda.init()
    W = device_weights(cfg, args.seed, torch)
    m = binding.Model(cfg, W, batch=B, capacity=P + n_new)
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed + 1)
    prompt = torch.randint(0, V, (B, P), generator=g, device="cuda", dtype=torch.int32)
    m.encode_prompt(prompt[:, :P - 1].contiguous())
    first = prompt[:, P - 1].contiguous()
    out = torch.empty((B, n_new), dtype=torch.int32, device="cuda")
    logits = torch.empty((B, V), dtype=torch.float32, device="cuda")
    names = list(binding.TIMERS)
    binding.timer_enable(names)
    for _ in range(args.warmup):
        m.ar_generate(first, n_new, out, logits)
        m.set_kv_length(P - 1)
    torch.cuda.synchronize()
    warm = {n: binding.timer_read(n) for n in names}
    binding.timer_enable([])
    dominant = max(names, key=lambda n: warm[n][0]) if args.warmup else "head_gemm"
    binding.timer_enable([dominant])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        m.ar_generate(first, n_new, out, logits)
        m.set_kv_length(P - 1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms, dom_n = binding.timer_read(dominant)
    binding.timer_enable(names)
    m.ar_generate(first, n_new, out, logits)
    m.set_kv_length(P - 1)
    torch.cuda.synchronize()
    kern = {}
    for n in names:
        ms, cnt = binding.timer_read(n)
        kern[n] = {"total_ms": round(ms, 3), "launches": cnt,
                   "avg_ms": round(ms / cnt, 5) if cnt else None}
    binding.timer_enable([])
    # one new token per sequence per launch; attention over the mean context
    acfg = dict(cfg, canvas=1)
    P_mean = P - 1 + n_new // 2
    roof = roofline(dominant, dom_ms / dom_n, acfg, B, P_mean, 1)
    roof["timed_launches"] = dom_n
    # up to 16 new tokens the head runs as the few-row decode kernel
    if dominant == "head_gemm" and B <= 16:
        roof["traffic"], roof["traffic_source"] = measured_traffic(
            dominant, f"ar_b{B}_{args.config}", source="gemm_decode.hip")
    else:
        roof["traffic"], roof["traffic_source"] = None, None
    per_kernel = {n: dict(kern[n], **({k: v for k, v in roofline(n, kern[n]["avg_ms"], acfg, B,
                                                                  P_mean, 1).items()
                                       if k in ("bound", "achieved", "unit", "frac")}
                                      if kern[n]["launches"] and n != "sampler" else {}))
                  for n in names}
    value = B * n_new * args.steps / wall
    out_json = {
        "metric": "AR decode tokens/s at 1 MI355X",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "ms_per_token": round(wall / (args.steps * n_new) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic (random-init N(0,0.02) weights, uniform random prompt tokens)",
        "config": {"workload": (f"ar-{args.config}: {cfg['n_layers']} layer(s) d{cfg['d_model']} "
                                f"{cfg['n_heads']}q/{cfg['n_kv_heads']}kv x{cfg['head_dim']}, "
                                f"{cfg['n_experts']} experts top-{cfg['top_k']} d_ff {cfg['d_ff']}, "
                                f"vocab {V}; greedy decoding of {n_new} tokens per sequence after "
                                f"a {P}-token prompt, batch {B}"),
                   "global_batch": B, "seq_len": P + n_new, "parallelism": "none (1 GPU)"},
        "kernels": per_kernel,
        "roofline": roof,
    }
    if args.copy_probe:
        copy_probe(torch)
    oracle_fits = cfg["n_layers"] == 1 and P <= 4096
    if args.no_cpu_baseline or not oracle_fits:
        out_json["cpu_baseline"] = None
    else:
        # the oracle decodes sequences one by one: one sequence is the sample
        out_json["cpu_baseline"] = cpu_baseline_ar(cfg, W, prompt[:1].cpu().numpy().astype(np.int64),
                                                   1)
    print(json.dumps(out_json), flush=True)


def cpu_baseline_train(cfg, W, prompt, clean, rate, seed):
    """The CPU oracle's training-side forward (float64 numpy model, C
    corruption), timed on this host after an untimed prompt encode."""
    import numpy as np
    from oracle import model as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    host = {"embed": W["embed"].float().cpu().numpy(), "w_sc": W["w_sc"].float().cpu().numpy(),
            "final_norm": W["final_norm"].cpu().numpy().astype(np.float64), "layers": []}
    for lw in W["layers"]:
        host["layers"].append({k: v.float().cpu().numpy() for k, v in lw.items()
                               if not k.startswith("s_")})
    B, N = clean.shape
    cache = om.KVCache(cfg, B)
    om.encode(prompt, host, cfg, cache)
    t0 = time.perf_counter()
    om.train_forward(clean, rate, seed, 0, host, cfg, cache)
    t1 = time.perf_counter()
    return {"value": round(B * N / (t1 - t0), 4), "unit": "canvas tokens/s",
            "cores": int(threads), "kind": "oracle",
            "sample": (f"one training-side forward of {B}x{N} canvas tokens after a "
                       f"{prompt.shape[1]}-token prompt ({(t1 - t0):.2f} s, float64 numpy, "
                       f"{threads} BLAS threads)")}


def bench_train(args):
    """The training-side forward: one step = dg_train_forward of every canvas
    of the batch at corruption rate --rate over the encoded prompt."""
    import numpy as np
    import torch

    from discrete_text_diffusion_denoise_amd import binding, synthetic

    shape = synthetic.SHAPES[args.config]
    over = {"n_layers": args.layers} if args.layers else {}
    cfg = synthetic.model_config(args.config, **over)
    if cfg.get("expert_dtype"):
        raise SystemExit("--mode train runs the bf16 configurations")
    B, N, V, P = shape["batch"], cfg["canvas"], cfg["vocab"], shape["prompt"]
    torch.cuda.init()
    W = device_weights(cfg, args.seed, torch)
    m = binding.Model(cfg, W, batch=B, capacity=P + N)
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed + 1)
    prompt = torch.randint(0, V, (B, P), generator=g, device="cuda", dtype=torch.int32)
    clean = torch.randint(0, V, (B, N), generator=g, device="cuda", dtype=torch.int32)
    rate = torch.full((B,), float(args.rate), dtype=torch.float32, device="cuda")
    m.encode_prompt(prompt)
    x = torch.empty((B, N), dtype=torch.int32, device="cuda")
    logits = torch.empty((B, N, V), dtype=torch.float32, device="cuda")
    loss = torch.empty((B, N), dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    names = list(binding.TIMERS)
    binding.timer_enable(names)
    for w in range(args.warmup):
        m.train_forward(clean, rate, args.seed, w, x, logits, loss, mean)
    torch.cuda.synchronize()
    warm = {n: binding.timer_read(n) for n in names}
    binding.timer_enable([])
    dominant = max(names, key=lambda n: warm[n][0]) if args.warmup else "head_gemm"
    hits = expert_hits(m, cfg, x, torch)
    cfg["experts_hit"] = float(np.mean(hits))
    binding.timer_enable([dominant])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        m.train_forward(clean, rate, args.seed, args.warmup + s_, x, logits, loss, mean)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms, dom_n = binding.timer_read(dominant)
    binding.timer_enable(names)
    m.train_forward(clean, rate, args.seed, 0, x, logits, loss, mean)
    torch.cuda.synchronize()
    kern = {}
    for n in names:
        ms, cnt = binding.timer_read(n)
        kern[n] = {"total_ms": round(ms, 3), "launches": cnt,
                   "avg_ms": round(ms / cnt, 5) if cnt else None}
    binding.timer_enable([])
    roof = roofline(dominant, dom_ms / dom_n, cfg, B, P, 1)
    roof["timed_launches"] = dom_n
    roof["traffic"], roof["traffic_source"] = measured_traffic(dominant, args.config)
    per_kernel = {n: dict(kern[n], **({k: v for k, v in roofline(n, kern[n]["avg_ms"], cfg, B, P,
                                                                  1).items()
                                       if k in ("bound", "achieved", "unit", "frac")}
                                      if kern[n]["launches"] else {}))
                  for n in names}
    value = B * N * args.steps / wall
    out = {
        "metric": "training-forward canvas tokens/s at 1 MI355X",
        "value": round(value, 2),
        "unit": "canvas tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"] + ("+fp8-experts" if cfg.get("expert_dtype") == "fp8" else ""),
        "data": "synthetic (random-init N(0,0.02) weights, uniform random prompt and clean tokens)",
        "config": {"workload": (f"train-{args.config}: {cfg['n_layers']} layer(s) "
                                f"d{cfg['d_model']}, vocab {V}, prompt {P}, canvas {N}, batch {B}; "
                                f"one step = corruption at rate {args.rate:g} + denoiser forward "
                                f"+ cross-entropy at the clean tokens"),
                   "global_batch": B, "seq_len": P + N, "parallelism": "none (1 GPU)",
                   "mean_loss": float(mean.cpu().numpy()[0])},
        "experts_hit_per_layer": {"min": min(hits), "mean": round(float(np.mean(hits)), 2),
                                  "max": max(hits), "of": cfg["n_experts"]},
        "kernels": per_kernel,
        "roofline": roof,
    }
    oracle_fits = cfg["n_layers"] == 1 and B == 1 and P <= 4096
    if args.no_cpu_baseline or not oracle_fits:
        out["cpu_baseline"] = None
    else:
        out["cpu_baseline"] = cpu_baseline_train(
            cfg, W, prompt.cpu().numpy().astype(np.int64), clean.cpu().numpy().astype(np.int32),
            np.full(B, args.rate, np.float32), args.seed)
    print(json.dumps(out), flush=True)


def bench_attn(args):
    """The attention block alone: dg_stage_attention of the configuration's B
    canvases of N tokens over a synthetic cache of P context keys per
    sequence (N(0, 4) keys, N(0, 1) values, bf16), one layer of the
    configuration's attention shape.  value = algorithmic FLOP/s of the
    attention kernel and its split merge (4 B N (P + N) Hq dh per launch),
    timed by the library's HIP events on the launch stream."""
    import torch

    from discrete_text_diffusion_denoise_amd import binding, synthetic

    shape = synthetic.SHAPES[args.config]
    # the attention block's shapes; a small vocabulary and expert set (unused)
    cfg = synthetic.model_config(args.config, n_layers=1, vocab=1024, n_experts=8, top_k=2,
                                 expert_dtype=None)
    B, P, N = shape["batch"], shape["prompt"], cfg["canvas"]
    Hq, dh, d = cfg["n_heads"], cfg["head_dim"], cfg["d_model"]
    torch.cuda.init()
    W = device_weights(cfg, args.seed, torch)
    m = binding.Model(cfg, W, batch=B, capacity=P + N)
    K, V = m.kv_tensors()
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed + 1)
    K[0, :, :, :P] = (2.0 * torch.randn(K[0, :, :, :P].shape, generator=g, device="cuda")).to(K.dtype)
    V[0, :, :, :P] = torch.randn(V[0, :, :, :P].shape, generator=g, device="cuda").to(V.dtype)
    m.set_kv_length(P)
    h0 = torch.randn((B * N, d), generator=g, device="cuda", dtype=torch.float32)
    h = h0.clone()
    for _ in range(args.warmup):
        h.copy_(h0)
        m.stage_attention(0, h, N, False)
    torch.cuda.synchronize()
    binding.timer_enable(["attention"])
    t0 = time.perf_counter()
    for _ in range(args.steps):
        h.copy_(h0)
        m.stage_attention(0, h, N, False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms, n = binding.timer_read("attention")
    binding.timer_enable([])
    flops = 4.0 * B * N * (P + N) * Hq * dh
    avg = ms / n
    ach = flops / (avg * 1e-3) / 1e12
    roof = roofline("attention", avg, cfg, B, P, 1)
    roof["timed_launches"] = n
    out = {
        "metric": "attention TFLOP/s at 1 MI355X",
        "value": round(ach, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic (N(0,4) keys, N(0,1) values, N(0,1) residual rows, random-init weights)",
        "config": {"workload": (f"attn-{args.config}: attention block of {B} canvas(es) of {N} "
                                f"tokens over {P} cached keys each, {Hq}q/{cfg['n_kv_heads']}kv "
                                f"x{dh}, d {d}; one step = one dg_stage_attention (projections, "
                                f"RoPE, attention, output projection)"),
                   "global_batch": B, "seq_len": P + N, "parallelism": "none (1 GPU)"},
        "attention_avg_ms": round(avg, 5),
        "roofline": roof,
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_moe(args):
    """The mixture-of-experts half alone: dg_stage_moe of the configuration's
    B canvases of N tokens (N(0, 1) residual rows) through one layer of its
    expert shape, weights drawn and quantised as in the full bench.  value =
    algorithmic HBM GB/s of the two expert products together (the weights of
    every expert the routes hit, read once, plus the activations), timed by
    the library's HIP events on the launch stream.

    --router-skew injects the router logits z = N(0, 1) + 0.5 on a seeded set
    of 13 hot experts (about 10 % of 128): the router rows are the first E unit
    vectors, and a token's first E features are its z (the rest N(0, 1)), so
    its logits after the RMSNorm are z / rms(row) -- a positive scale that
    keeps the token's top-k exactly that of z."""
    import torch

    from discrete_text_diffusion_denoise_amd import binding, synthetic

    shape = synthetic.SHAPES[args.config]
    cfg = synthetic.model_config(args.config, n_layers=1, vocab=1024)
    B, N, d = shape["batch"], cfg["canvas"], cfg["d_model"]
    torch.cuda.init()
    W = device_weights(cfg, args.seed, torch)
    E = cfg["n_experts"]
    hot = None
    if args.router_skew:
        W["layers"][0]["w_router"] = torch.eye(E, d, device="cuda").to(W["layers"][0]["w_router"].dtype)
        hot = torch.randperm(E, generator=torch.Generator().manual_seed(args.seed + 7))[:13]
    m = binding.Model(cfg, W, batch=B, capacity=N + 16)
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed + 1)
    T = B * N
    h0 = torch.randn((T, d), generator=g, device="cuda", dtype=torch.float32)
    if hot is not None:
        h0[:, hot.to("cuda")] += 0.5
    h = h0.clone()
    route = torch.zeros((T, cfg["top_k"]), dtype=torch.int32, device="cuda")
    gates = torch.zeros((T, cfg["top_k"]), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        h.copy_(h0)
        m.stage_moe(0, h, route, gates)
    torch.cuda.synchronize()
    hit = int(torch.unique(route).numel())
    cfg["experts_hit"] = hit
    load = torch.bincount(route.reshape(-1).long(), minlength=E).float()
    load_stats = {"max": int(load.max()), "mean": round(float(load.mean()), 2),
                  "max_over_mean": round(float(load.max() / load.mean()), 3),
                  "hot_mean": round(float(load[hot].mean()), 2) if hot is not None else None,
                  "cold_mean": (round(float(load[[e for e in range(E) if e not in set(hot.tolist())]].mean()), 2)
                                if hot is not None else None)}
    binding.timer_enable(["moe_gateup", "moe_down"])
    t0 = time.perf_counter()
    for _ in range(args.steps):
        h.copy_(h0)
        m.stage_moe(0, h, route, gates)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernels, total_bytes, total_ms = {}, 0.0, 0.0
    for name in ("moe_gateup", "moe_down"):
        ms, n = binding.timer_read(name)
        avg = ms / n
        r = roofline(name, avg, cfg, B, 0, 1)
        kernels[name] = {"avg_ms": round(avg, 5), "launches": n, "achieved": r["achieved"],
                         "unit": r["unit"], "frac": r["frac"], "bytes_per_launch": r["bytes_per_launch"]}
        total_bytes += r["bytes_per_launch"]
        total_ms += avg
    binding.timer_enable([])
    if args.copy_probe:
        copy_probe(torch)
    # measured HBM bytes per launch, from the committed counter summaries of
    # this workload (null when absent or taken on an older kernel source)
    src = "moe_mx.hip" if cfg.get("expert_dtype") in ("fp8", "mxfp4") else "moe.hip"
    traffic = 0.0
    for name in kernels:
        t, where = measured_traffic(name, "moe_" + args.config + ("_skew" if hot is not None else ""),
                                    source=src)
        kernels[name]["traffic"] = round(t) if t is not None else None
        kernels[name]["traffic_source"] = where
        traffic = traffic + t if (t is not None and traffic is not None) else None
    ach = total_bytes / (total_ms * 1e-3) / 1e9
    fmt = {"fp8": "E4M3 weights, per-row scales", "mxfp4": "MXFP4 weights"}.get(
        cfg.get("expert_dtype"), cfg["dtype"] + " weights")
    out = {
        "metric": "MoE expert GEMM GB/s at 1 MI355X",
        "value": round(ach, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"] + {"fp8": "+fp8-experts", "mxfp4": "+mxfp4-experts"}.get(
            cfg.get("expert_dtype"), ""),
        "data": "synthetic (N(0,1) residual rows, random-init N(0,0.02) weights)",
        "config": {"workload": (f"moe-{args.config}{'-skew' if hot is not None else ''}: MoE half of "
                                f"{B} canvas(es) of {N} tokens, "
                                f"d {d}, {cfg['n_experts']} experts top-{cfg['top_k']}, d_ff "
                                f"{cfg['d_ff']} ({fmt}); one step = one dg_stage_moe (RMSNorm, "
                                f"router, routing, both expert products, combine)"),
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "experts_hit": hit,
        "expert_load": load_stats,
        "router": ("injected logits N(0,1) + 0.5 on 13 hot experts" if hot is not None
                   else "random router weights, N(0,1) rows"),
        "kernels": kernels,
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": round(traffic) if traffic else None,
                     "kernel": "moe_gateup+moe_down", "bytes_per_launch": total_bytes,
                     "avg_launch_ms": round(total_ms, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the kernels run on one GPU's share at full shape).", file=sys.stderr)
        sys.exit(2)
    if args.mode == "ar":
        bench_ar(args)
        return
    if args.mode == "moe":
        bench_moe(args)
        return
    if args.mode == "train":
        bench_train(args)
        return
    if args.mode == "attn":
        bench_attn(args)
        return
    out = bench_diffusion(args, args.config, args.layers, args.steps, args.warmup,
                          not args.no_cpu_baseline)
    if args.config == "layer" and not args.layers and not args.no_stack:
        # the full denoise step's 30-layer stack, timed in the same run (its
        # own line's essentials under one key)
        st = bench_diffusion(args, "stack", None, args.stack_steps, 1, False)
        out["stack"] = {k: st[k] for k in ("metric", "value", "unit", "ms_per_step",
                                           "denoise_step_ms", "canvas_tokens_per_s_at_12_rounds",
                                           "prefill", "trajectory",
                                           "kernels", "roofline",
                                           "experts_hit_per_layer", "fraction_check")}
        out["stack"]["steps"] = args.stack_steps
        out["stack"]["workload"] = st["config"]["workload"]
        out["stack"]["rounds_per_block"] = st["config"]["rounds_per_block"]
        out["stack"]["sampler"] = st["config"]["sampler"]
    print(json.dumps(out), flush=True)


def expert_hits(m, cfg, canvas, torch):
    """Distinct experts that receive at least one token, per layer, in one
    denoising round of `canvas` without self-conditioning (run as the chain
    of its stage calls, which is the step's own computation)."""
    B, N = canvas.shape
    h = torch.empty((B * N, cfg["d_model"]), dtype=torch.float32, device="cuda")
    route = torch.empty((B * N, cfg["top_k"]), dtype=torch.int32, device="cuda")
    m.stage_input(canvas, h)
    hits = []
    for l in range(cfg["n_layers"]):
        m.stage_attention(l, h, N, False)
        m.stage_moe(l, h, route)
        hits.append(int(torch.unique(route).numel()))
    return hits


def bench_diffusion(args, config, layers, steps, warmup, want_cpu):
    """One configuration of the block loop: returns the JSON dict."""
    import numpy as np
    import torch

    from discrete_text_diffusion_denoise_amd import binding, synthetic

    shape = synthetic.SHAPES[config]
    over = {"n_layers": layers} if layers else {}
    cfg = synthetic.model_config(config, **over)
    cfg["sampler_top_k"] = args.top_k
    # the full-distribution sampler is bound by its binary32 arithmetic; in
    # the block loop of bf16 models it also writes the next round's
    # self-conditioning weights
    cfg["sampler_alu"] = args.top_k == 0
    cfg["sampler_probs"] = args.top_k == 0 and cfg["dtype"] == "bf16"
    B, N, V, P = shape["batch"], cfg["canvas"], cfg["vocab"], shape["prompt"]
    # consecutive blocks per step, each committed before the next (the cache
    # is rewound to the prompt after the last)
    nb = shape.get("blocks", 1)
    torch.cuda.init()
    W = device_weights(cfg, args.seed, torch)
    m = binding.Model(cfg, W, batch=B, capacity=P + (nb + 1) * N, generate_ws=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed + 1)
    prompt = torch.randint(0, V, (B, P), generator=g, device="cuda", dtype=torch.int32)
    # the prompt encode (causal prefill of B x P tokens through every layer),
    # timed on its own (the second of two identical encodes, the cache rewound
    # between them): not part of a step
    m.encode_prompt(prompt)
    m.set_kv_length(0)
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    pe[0].record()
    m.encode_prompt(prompt)
    pe[1].record()
    torch.cuda.synchronize()
    prefill_ms = pe[0].elapsed_time(pe[1])
    params = synthetic.default_sampler_params(max_steps=48, seed=args.seed, selfcond_on=1,
                                              top_k=args.top_k,
                                              stop_tau=shape.get("stop_tau", 0.005),
                                              **shape.get("sampler", {}))
    block = torch.zeros((B, N), dtype=torch.int32, device="cuda")

    names = list(binding.TIMERS)
    # warmup, with every kernel timer on: picks the dominant kernel
    binding.timer_enable(names)
    for w in range(warmup):
        for k in range(nb):
            m.generate_block(params, w * nb + k, block)
        m.set_kv_length(P)
    torch.cuda.synchronize()
    warm = {n: binding.timer_read(n) for n in names}
    binding.timer_enable([])
    dominant = max(names, key=lambda n: warm[n][0]) if warmup else "head_gemm"
    # experts that receive tokens, per layer, in the first round of a block
    # (its starting canvas): the expert kernels' algorithmic bytes count the
    # weights of every hit expert once (routing of the random-init stack is
    # far from uniform, so a uniform-routing estimate would overstate them)
    start = torch.zeros((B, N), dtype=torch.int32, device="cuda")
    binding.canvas_init(params["seed"], 0, start, V)
    hits = expert_hits(m, cfg, start, torch)
    m.set_kv_length(P)
    cfg["experts_hit"] = float(np.mean(hits))

    # timed blocks: only the dominant kernel is bracketed by the library's
    # HIP events (on the stream it runs on); every other timer is off, since
    # each recorded event sits between two kernels
    binding.timer_enable([dominant])
    rounds = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        for k in range(nb):
            rounds += m.generate_block(params, (warmup + s) * nb + k, block)
        m.set_kv_length(P)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    dom_ms, dom_n = binding.timer_read(dominant)
    binding.timer_enable([])

    # per-kernel breakdown: one more block with every timer on, recording the
    # rounds' mean entropy and locked count (dg_generate_block_trace)
    binding.timer_enable(names)
    trace = torch.full((params["max_steps"], B, 2), float("nan"), dtype=torch.float32,
                       device="cuda")
    tr_steps = m.generate_block(params, warmup + steps, block, trace=trace)
    m.set_kv_length(P)
    torch.cuda.synchronize()
    tr = trace.cpu().numpy()
    pick = [t for t in (0, 1, 2, 4, 8, 16, 32, params["max_steps"] - 1) if t < tr_steps[0]]
    kern = {}
    for n in names:
        ms, cnt = binding.timer_read(n)
        kern[n] = {"total_ms": round(ms, 3), "launches": cnt,
                   "avg_ms": round(ms / cnt, 5) if cnt else None}
    binding.timer_enable([])

    # denoise-step latency: one self-conditioned dg_denoise_step + dg_sample_update
    logits = [torch.empty((B, N, V), dtype=torch.float32, device="cuda") for _ in range(2)]
    stats = [torch.zeros((B, N, 4), dtype=torch.float32, device="cuda") for _ in range(2)]
    canvas = torch.zeros((B, N), dtype=torch.int32, device="cuda")
    binding.canvas_init(params["seed"], 0, canvas, V)
    argmax = torch.zeros((B, N), dtype=torch.int32, device="cuda")
    lock = torch.zeros((B, N), dtype=torch.uint8, device="cuda")
    stop = torch.zeros(B, dtype=torch.int32, device="cuda")
    sws = binding.sampler_workspace(B, N)
    m.denoise_step(canvas, logits[0])
    binding.sample_update(params, 0, logits[0], canvas, argmax, lock, stats[0], stop, sws)
    reps = 11
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for j in range(1, reps + 1):
        stop.zero_()
        m.denoise_step(canvas, logits[j % 2], logits[(j - 1) % 2], stats[(j - 1) % 2],
                       top_k=args.top_k)
        binding.sample_update(params, j, logits[j % 2], canvas, argmax, lock, stats[j % 2], stop,
                              sws)
        ev[j].record()
    torch.cuda.synchronize()
    # median over the steps (each timed between consecutive events)
    step_ms = float(np.median([ev[j - 1].elapsed_time(ev[j]) for j in range(1, reps + 1)]))

    sc_tiles = -(-B * N // 256) * -(-cfg["d_model"] // 256)
    sc_splits = max(1, min(64, 256 // max(sc_tiles, 1)))
    sc_splits = (sc_splits // 8) * 8 if sc_splits >= 8 else sc_splits
    k_split = -(-(-(-V // sc_splits)) // 128) * 128
    sc_splits = -(-V // k_split)
    roof = roofline(dominant, dom_ms / dom_n, cfg, B, P, sc_splits)
    roof["timed_launches"] = dom_n
    roof["traffic"], roof["traffic_source"] = measured_traffic(dominant, config)
    per_kernel = {n: dict(kern[n], **({k: v for k, v in roofline(n, kern[n]["avg_ms"], cfg, B, P,
                                                                  sc_splits).items()
                                       if k in ("bound", "achieved", "unit", "frac")}
                                      if kern[n]["launches"] else {}))
                  for n in names}

    value = B * N * steps * nb / wall
    fracs = {n: v["frac"] for n, v in per_kernel.items() if "frac" in v}
    fracs["roofline"] = roof["frac"]
    over1 = sorted(n for n, f in fracs.items() if f > 1.0)
    if over1:
        print(f"bench.py: fraction of peak above 1 for {over1}: the byte or flop model is wrong",
              file=sys.stderr)
    out = {
        "metric": "canvas tokens/s at 1 MI355X",
        "value": round(value, 2),
        "unit": "canvas tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"] + {"fp8": "+fp8-experts", "mxfp4": "+mxfp4-experts"}.get(
            cfg.get("expert_dtype"), ""),
        "data": "synthetic (random-init N(0,0.02) weights, uniform random prompt tokens)",
        "config": {"workload": (f"{config}: {cfg['n_layers']} denoiser layer(s) d{cfg['d_model']} "
                                f"{cfg['n_heads']}q/{cfg['n_kv_heads']}kv x{cfg['head_dim']}, "
                                f"{cfg['n_experts']} experts top-{cfg['top_k']} d_ff {cfg['d_ff']}"
                                f"{ {'fp8': ' (E4M3 weights, per-row scales)', 'mxfp4': ' (MXFP4 weights)'}.get(cfg.get('expert_dtype'), '')}, "
                                f"vocab {V}, prompt {P}, canvas {N}, batch {B}; one step = one "
                                f"block (<=48 self-conditioned rounds + commit)"
                                + (f"; here one step = {nb} consecutive blocks, each committed "
                                   f"(context {P} .. {P + (nb - 1) * N})" if nb > 1 else "")),
                   "global_batch": B, "seq_len": P + N, "parallelism": "none (1 GPU)",
                   "rounds_per_block": float(np.mean(rounds)) if rounds else None,
                   "sampler": ((f"cumulative-entropy lock {params['lock_theta']:g}"
                                if params["lock_rule"] == 1 else
                                f"lock where max-probability > {params['lock_theta']:g}")
                               + f", T {params['temp_start']:g}->{params['temp_end']:g}, stop "
                               f"{params['stop_tau']:g} + stable"
                               + (f", top-{args.top_k} truncation" if args.top_k else ""))},
        "weights_cache": ("cold: a round streams both vocabulary products' E (2 x "
                          f"{2 * V * cfg['d_model'] / 1e9:.2f} GB) and every hit expert, far "
                          "more than the 256 MB last-level cache, so no weight is cache-warm "
                          "from one round to the next"),
        "prefill": {"ms": round(prefill_ms, 3), "tokens": B * P,
                    "note": "one causal prompt encode (the second of two), not part of the "
                            "timed steps"},
        "trajectory": {"canvas": 0, "rounds": pick,
                       "mean_entropy_nats": [round(float(tr[t, 0, 0]), 4) for t in pick],
                       "locked_fraction": [round(float(tr[t, 0, 1]) / N, 4) for t in pick],
                       "tokens_per_forward": round(N / float(np.mean(rounds)), 3) if rounds
                       else None},
        "denoise_step_ms": round(step_ms, 4),
        "canvas_tokens_per_s_at_12_rounds": (
            round(value * float(np.mean(rounds)) / 12.0, 1) if rounds else None),
        "kernels": per_kernel,
        "roofline": roof,
        "experts_hit_per_layer": {"min": min(hits), "mean": round(float(np.mean(hits)), 2),
                                  "max": max(hits), "of": cfg["n_experts"],
                                  "layers": len(hits)},
        "fraction_check": ("ok: every fraction of peak <= 1" if not over1 else
                           f"FAILED: above 1 for {over1}"),
    }
    if args.copy_probe and config == args.config:
        copy_probe(torch)
    # (not with --copy-probe: the calibration's own device copy would join the
    # copies the HBM counters are calibrated on)
    if config == args.config and not args.no_peaks and not args.copy_probe:
        pk = measured_peaks(torch)
        out["measured_peaks"] = pk
        ref = {"hbm": pk["hbm_read_gbs"], "mfma": pk["bf16_mfma_tflops"]}.get(roof["bound"])
        if ref:
            roof["frac_of_measured_peak"] = round(roof["achieved"] / ref, 4)
    oracle_fits = cfg["n_layers"] == 1 and B == 1 and P <= 4096
    if want_cpu and not oracle_fits:
        # the float64 oracle's prompt encode alone would run for many minutes
        out["cpu_baseline"] = None
        out["cpu_baseline_note"] = ("skipped: the oracle sample is defined for the one-layer, "
                                    "one-canvas workload")
    elif want_cpu:
        cpu_canvas = np.asarray(canvas.cpu().numpy(), dtype=np.int64)
        out["cpu_baseline"] = cpu_baseline(cfg, W, prompt.cpu().numpy().astype(np.int64),
                                           cpu_canvas, params, torch)
    else:
        out["cpu_baseline"] = None
    del m, W, logits, stats
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
