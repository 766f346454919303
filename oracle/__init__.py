"""CPU oracle of one denoising step of a block text-diffusion MoE model.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call, link or execute anything
under ``oracle/``.  The product path (the HIP library and its Python binding)
never does, and shares no code with it: no kernels, headers, helpers, tables
or constant generators.

  model.py    float64 numpy forward: embedding + self-conditioning (full or
              top-k truncated), causal and bidirectional attention over a KV
              cache, top-k SwiGLU MoE, tied head, prompt encode and block
              commit; the retained autoregressive mode (causal forward,
              one-token decode, greedy decoding); the training-side forward.
  sampler.c   binary32 sampler (statistics, Philox draw, lock rules, renoise,
              stop; top-k truncation; corruption and cross-entropy of the
              training forward) with every floating-point operation fixed,
              so that decisions can be compared bit for bit; sampler.py
              wraps it.
  quant.py    the 8-bit (E4M3, per-row scale) and MXFP4 (E2M1, E8M0 scale
              per 32) expert-weight formats.
  driver.py   the block loop: canvas init, denoise/sample rounds, commit.

Parity pins live in tests/test_oracle_*.py; every function has one (a
function without a pin would say "parity unpinned" in its docstring).
"""
