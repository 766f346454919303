"""ctypes binding of libdg.so (include/dg.h).

Argument marshalling only: torch provides device memory and the stream, every
step of the path runs in the library's HIP kernels.  Loading fails loudly if
the library has not been built (python -m discrete_text_diffusion_denoise_amd.build);
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdg.so")
_lib = None

DG_F32, DG_BF16, DG_FP8_E4M3, DG_MXFP4 = 0, 1, 2, 3
LOCK_MAXPROB, LOCK_CUMENT = 0, 1
STATUS = {0: "DG_OK", 1: "DG_ERR_ARG", 2: "DG_ERR_SHAPE", 3: "DG_ERR_DTYPE",
          4: "DG_ERR_CAPACITY", 5: "DG_ERR_NONFINITE", 6: "DG_ERR_HIP", 7: "DG_ERR_UNSUPPORTED"}


class DGError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("canvas", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_on", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("expert_dtype", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "moe_norm", "w_router", "w_gate", "w_up",
                 "w_down", "s_gate", "s_up", "s_down", "x_gate", "x_up", "x_down")]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("embed_t", ctypes.c_void_p),
                ("w_sc", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerWeights)), ("embed_head", ctypes.c_void_p)]


class SamplerParams(ctypes.Structure):
    _fields_ = [("lock_rule", ctypes.c_int32), ("lock_theta", ctypes.c_float),
                ("temp_start", ctypes.c_float), ("temp_end", ctypes.c_float),
                ("stop_tau", ctypes.c_float), ("require_stable", ctypes.c_int32),
                ("max_steps", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("selfcond_on", ctypes.c_int32), ("top_k", ctypes.c_int32)]


# exported symbol -> (restype, argtypes)
_P, _I, _U64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
_SIGS = {
    "dg_status_string": (ctypes.c_char_p, [_I]),
    "dg_last_error": (ctypes.c_char_p, []),
    "dg_model_create": (_I, [_P, _P, _P]),
    "dg_model_destroy": (None, [_P]),
    "dg_embed_transpose": (_I, [_P, _P, _P, _P]),
    "dg_embed_head_bytes": (_I, [_P, _P]),
    "dg_embed_head": (_I, [_P, _P, _P, _P]),
    "dg_quantize_fp8": (_I, [_P, _I, ctypes.c_int64, _I, _P, _P, _P]),
    "dg_quantize_mxfp4": (_I, [_P, _I, ctypes.c_int64, _I, _P, _P, _P]),
    "dg_kv_bytes": (_I, [_P, _I, _I, _P]),
    "dg_kv_create": (_I, [_P, _I, _I, _P, _P]),
    "dg_kv_destroy": (None, [_P]),
    "dg_kv_length": (_I, [_P, _P]),
    "dg_kv_set_length": (_I, [_P, _I]),
    "dg_workspace_bytes": (_I, [_P, _I, _P]),
    "dg_sampler_workspace_bytes": (_I, [_I, _I, _P]),
    "dg_encode_prompt": (_I, [_P, _P, _I, _P, _I, _P, _SZ, _P]),
    "dg_denoise_step": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "dg_denoise_step_topk": (_I, [_P, _P, _I, _P, _P, _P, _I, _P, _P, _SZ, _P]),
    "dg_sample_update": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dg_sample_update_static": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "dg_sample_update_probs": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                    _SZ, _P]),
    "dg_stage_probs": (_I, [_I, _I, _I, _P, _P, _P, _P]),
    "dg_canvas_init": (_I, [_U64, _I, _I, _I, _I, _P, _P]),
    "dg_commit_block": (_I, [_P, _P, _I, _P, _P, _SZ, _P]),
    "dg_ar_decode_step": (_I, [_P, _P, _I, _P, _P, _P, _SZ, _P]),
    "dg_argmax_rows": (_I, [_I, _I, _P, _P, _P]),
    "dg_ar_generate": (_I, [_P, _P, _I, _P, _I, _P, _P, _P, _SZ, _P]),
    "dg_corrupt": (_I, [ctypes.c_uint64, _I, _I, _I, _I, _P, _P, _P, _P]),
    "dg_xent": (_I, [_I, _I, _P, _P, _P, _P, _P]),
    "dg_train_forward": (_I, [_P, _P, _I, _P, _P, ctypes.c_uint64, _I, _P, _P, _P, _P, _P, _SZ,
                              _P]),
    "dg_generate_workspace_bytes": (_I, [_P, _I, _P]),
    "dg_generate_block": (_I, [_P, _P, _I, _P, _I, _P, _P, _P, _SZ, _P]),
    "dg_generate_block_trace": (_I, [_P, _P, _I, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "dg_stage_input": (_I, [_P, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "dg_stage_input_topk": (_I, [_P, _I, _P, _P, _I, _P, _P, _SZ, _P]),
    "dg_stage_attention": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "dg_stage_moe": (_I, [_P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "dg_stage_head": (_I, [_P, _I, _P, _P, _P, _SZ, _P]),
    "dg_stage_head_rowmax": (_I, [_P, _I, _P, _P, _P, _P, _SZ, _P]),
    "dg_timer_enable": (_I, [ctypes.c_uint32]),
    "dg_timer_read": (_I, [_I, _P, _P]),
    "dg_measure_peaks": (_I, [_P, _SZ, _P, _P, _P]),
}

TIMERS = {"head_gemm": 0, "selfcond_gemm": 1, "moe_gateup": 2, "moe_down": 3, "attention": 4,
          "sampler": 5}
EXPORTED = tuple(_SIGS)


def lib():
    """The loaded library; raises if libdg.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m discrete_text_diffusion_denoise_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise DGError(status, lib().dg_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous CUDA tensors"
        return ctypes.c_void_p(t.data_ptr())
    return t


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def sampler_params(p: dict) -> SamplerParams:
    return SamplerParams(int(p["lock_rule"]), float(p["lock_theta"]), float(p["temp_start"]),
                         float(p["temp_end"]), float(p["stop_tau"]), int(p["require_stable"]),
                         int(p["max_steps"]), int(p["seed"]), int(p.get("selfcond_on", 1)),
                         int(p.get("top_k", 0)))


# ------------------------------------------------------------------ model handle

class Model:
    """Device weights + dg_model handle + KV cache + workspace.

    weights: dict of numpy arrays as produced by synthetic.make_weights (or
    torch CUDA tensors of the right dtype); cfg: synthetic.model_config dict."""

    def __init__(self, cfg: dict, weights: dict, batch: int, capacity: int,
                 device: str = "cuda:0", generate_ws: bool = False):
        self.cfg = cfg
        self.batch = batch
        self.device = torch.device(device)
        self.dtype = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
        L = lib()

        def dev(a, dtype=None):
            if isinstance(a, torch.Tensor):
                return a.to(self.device).contiguous()
            t = torch.from_numpy(np.ascontiguousarray(a))
            return t.to(self.device).to(dtype or self.dtype).contiguous()

        self.w = {"embed": dev(weights["embed"]), "w_sc": dev(weights["w_sc"]),
                  "final_norm": dev(weights["final_norm"], torch.float32)}
        # 8-bit experts: w_gate / w_up / w_down hold E4M3 codes (uint8) and
        # s_gate / s_up / s_down their per-row fp32 scales
        # MXFP4 experts: w_* hold packed E2M1 codes (uint8 [E][R][K/2]) and
        # x_gate / x_up / x_down the E8M0 scale codes ([K/64][E*R][2], uint8)
        fp8 = cfg.get("expert_dtype") == "fp8"
        fp4 = cfg.get("expert_dtype") == "mxfp4"

        def ldtype(k):
            if k.endswith("norm") or k.startswith("s_"):
                return torch.float32
            if (fp8 or fp4) and k in ("w_gate", "w_up", "w_down"):
                return torch.uint8
            if k.startswith("x_"):
                return torch.uint8
            return None

        self.lw = []
        for lw in weights["layers"]:
            d = {k: dev(v, ldtype(k)) for k, v in lw.items()}
            self.lw.append(d)
        c = Config(cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"],
                   cfg["head_dim"], cfg["n_experts"], cfg["top_k"], cfg["d_ff"], cfg["vocab"],
                   cfg["canvas"], DG_BF16 if cfg["dtype"] == "bf16" else DG_F32,
                   int(cfg["rope_on"]), float(cfg["rope_theta"]), float(cfg["rms_eps"]),
                   DG_FP8_E4M3 if fp8 else (DG_MXFP4 if fp4 else 0))
        self._cfg_struct = c
        layer_arr = (LayerWeights * cfg["n_layers"])()
        for i, d in enumerate(self.lw):
            for k in ("attn_norm", "wq", "wk", "wv", "wo", "moe_norm", "w_router", "w_gate",
                      "w_up", "w_down"):
                setattr(layer_arr[i], k, d[k].data_ptr())
            if fp8:
                for k in ("s_gate", "s_up", "s_down"):
                    setattr(layer_arr[i], k, d[k].data_ptr())
            if fp4:
                for k in ("x_gate", "x_up", "x_down"):
                    setattr(layer_arr[i], k, d[k].data_ptr())
        self._layer_arr = layer_arr
        self.w["embed_t"] = torch.empty((cfg["d_model"], cfg["vocab"]), dtype=self.dtype,
                                        device=self.device)
        w = Weights(self.w["embed"].data_ptr(), self.w["embed_t"].data_ptr(),
                    self.w["w_sc"].data_ptr(), self.w["final_norm"].data_ptr(), layer_arr, None)
        h = ctypes.c_void_p()
        _check(L.dg_model_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)))
        # blocked models take the head's operand prepared once (the weight
        # table is copied at create, so the model is created again with it)
        nb = ctypes.c_size_t()
        _check(L.dg_embed_head_bytes(h, ctypes.byref(nb)))
        if nb.value:
            self.w["embed_head"] = torch.empty(nb.value, dtype=torch.uint8, device=self.device)
            w.embed_head = self.w["embed_head"].data_ptr()
            L.dg_model_destroy(h)
            h = ctypes.c_void_p()
            _check(L.dg_model_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)))
            _check(L.dg_embed_head(h, _ptr(self.w["embed"]), _ptr(self.w["embed_head"]),
                                   _stream()))
        self._w_struct = w
        self.handle = h
        _check(L.dg_embed_transpose(h, _ptr(self.w["embed"]), _ptr(self.w["embed_t"]),
                                    _stream()))
        # KV cache
        nb = ctypes.c_size_t()
        _check(L.dg_kv_bytes(h, batch, capacity, ctypes.byref(nb)))
        self.kv_buf = torch.empty(nb.value, dtype=torch.uint8, device=self.device)
        kv = ctypes.c_void_p()
        _check(L.dg_kv_create(h, batch, capacity, _ptr(self.kv_buf), ctypes.byref(kv)))
        self.kv = kv
        self.capacity = capacity
        # workspace
        ws = ctypes.c_size_t()
        if generate_ws:
            _check(L.dg_generate_workspace_bytes(h, batch, ctypes.byref(ws)))
        else:
            _check(L.dg_workspace_bytes(h, batch, ctypes.byref(ws)))
        self.ws = torch.empty(ws.value, dtype=torch.uint8, device=self.device)

    def __del__(self):
        try:
            if getattr(self, "kv", None):
                lib().dg_kv_destroy(self.kv)
            if getattr(self, "handle", None):
                lib().dg_model_destroy(self.handle)
        except Exception:
            pass

    # ---- KV
    @property
    def kv_length(self) -> int:
        n = ctypes.c_int32()
        _check(lib().dg_kv_length(self.kv, ctypes.byref(n)))
        return n.value

    def set_kv_length(self, n: int):
        _check(lib().dg_kv_set_length(self.kv, int(n)))

    def kv_tensors(self):
        """(K, V) views [n_layers, B, Hkv, capacity, dh] of the cache buffer."""
        c = self.cfg
        shape = (c["n_layers"], self.batch, c["n_kv_heads"], self.capacity, c["head_dim"])
        flat = self.kv_buf.view(self.dtype)
        n = int(np.prod(shape))
        return flat[:n].view(shape), flat[n:2 * n].view(shape)

    # ---- the path (names follow include/dg.h)
    def encode_prompt(self, tokens: torch.Tensor, stream=None):
        B, P = tokens.shape
        _check(lib().dg_encode_prompt(self.handle, self.kv, B, _ptr(tokens), P, _ptr(self.ws),
                                      self.ws.numel(), _stream(stream)))

    def denoise_step(self, canvas, logits, prev_logits=None, prev_stats=None, stream=None,
                     top_k: int = 0):
        """dg_denoise_step (top_k > 0: dg_denoise_step_topk, the self-conditioning
        truncated to each position's top_k previous logits)."""
        if top_k:
            _check(lib().dg_denoise_step_topk(self.handle, self.kv, canvas.shape[0], _ptr(canvas),
                                              _ptr(prev_logits), _ptr(prev_stats), int(top_k),
                                              _ptr(logits), _ptr(self.ws), self.ws.numel(),
                                              _stream(stream)))
            return
        _check(lib().dg_denoise_step(self.handle, self.kv, canvas.shape[0], _ptr(canvas),
                                     _ptr(prev_logits), _ptr(prev_stats), _ptr(logits),
                                     _ptr(self.ws), self.ws.numel(), _stream(stream)))

    def ar_decode_step(self, tokens, logits, stream=None):
        """dg_ar_decode_step: tokens [B] int32 -> logits [B, V] f32; len += 1."""
        _check(lib().dg_ar_decode_step(self.handle, self.kv, tokens.shape[0], _ptr(tokens),
                                       _ptr(logits), _ptr(self.ws), self.ws.numel(),
                                       _stream(stream)))

    def ar_generate(self, first, n_new: int, out, logits, stream=None):
        """dg_ar_generate: greedy decoding of n_new tokens per sequence from
        first [B] into out [B, n_new] int32; logits [B, V] f32 scratch."""
        _check(lib().dg_ar_generate(self.handle, self.kv, first.shape[0], _ptr(first), int(n_new),
                                    _ptr(out), _ptr(logits), _ptr(self.ws), self.ws.numel(),
                                    _stream(stream)))

    def train_forward(self, clean, rate, seed: int, step: int, corrupted, logits, loss,
                      mean=None, stream=None):
        """dg_train_forward: clean [B, N] int32, rate [B] f32 -> corrupted [B, N],
        logits [B, N, V], loss [B, N] f32, mean [1] f32 (optional)."""
        _check(lib().dg_train_forward(self.handle, self.kv, clean.shape[0], _ptr(clean),
                                      _ptr(rate), int(seed), int(step), _ptr(corrupted),
                                      _ptr(logits), _ptr(loss),
                                      _ptr(mean) if mean is not None else None,
                                      _ptr(self.ws), self.ws.numel(), _stream(stream)))

    def commit_block(self, block, stream=None):
        _check(lib().dg_commit_block(self.handle, self.kv, block.shape[0], _ptr(block),
                                     _ptr(self.ws), self.ws.numel(), _stream(stream)))

    def generate_block(self, params: dict, block_index: int, block_out, stream=None,
                       trace=None):
        """dg_generate_block; with `trace` (float32 [max_steps, batch, 2] on
        the device) dg_generate_block_trace, which also records each round's
        mean entropy and locked count per canvas."""
        steps = (ctypes.c_int32 * self.batch)()
        sp = sampler_params(params)
        if trace is None:
            _check(lib().dg_generate_block(self.handle, self.kv, self.batch, ctypes.byref(sp),
                                           int(block_index), _ptr(block_out), steps,
                                           _ptr(self.ws), self.ws.numel(), _stream(stream)))
        else:
            if tuple(trace.shape) != (int(params["max_steps"]), self.batch, 2) or \
                    trace.dtype != torch.float32:
                raise ValueError("trace must be float32 [max_steps, batch, 2]")
            _check(lib().dg_generate_block_trace(self.handle, self.kv, self.batch,
                                                 ctypes.byref(sp), int(block_index),
                                                 _ptr(block_out), steps, _ptr(trace),
                                                 _ptr(self.ws), self.ws.numel(), _stream(stream)))
        return list(steps)

    # ---- stages
    def stage_input(self, canvas, h, prev_logits=None, prev_stats=None, stream=None):
        _check(lib().dg_stage_input(self.handle, canvas.shape[0], _ptr(canvas),
                                    _ptr(prev_logits), _ptr(prev_stats), _ptr(h), _ptr(self.ws),
                                    self.ws.numel(), _stream(stream)))

    def stage_input_topk(self, canvas, h, prev_logits, top_k: int, stream=None):
        """dg_stage_input_topk: the input stage with top_k-truncated self-conditioning."""
        _check(lib().dg_stage_input_topk(self.handle, canvas.shape[0], _ptr(canvas),
                                         _ptr(prev_logits), int(top_k), _ptr(h), _ptr(self.ws),
                                         self.ws.numel(), _stream(stream)))

    def stage_attention(self, layer, h, n, causal, stream=None):
        _check(lib().dg_stage_attention(self.handle, self.kv, int(layer), self.batch, int(n),
                                        int(causal), _ptr(h), _ptr(self.ws), self.ws.numel(),
                                        _stream(stream)))

    def stage_moe(self, layer, h, route=None, gates=None, stream=None):
        _check(lib().dg_stage_moe(self.handle, int(layer), h.shape[0], _ptr(h), _ptr(route),
                                  _ptr(gates), _ptr(self.ws), self.ws.numel(), _stream(stream)))

    def stage_head(self, h, logits, stream=None):
        _check(lib().dg_stage_head(self.handle, h.shape[0], _ptr(h), _ptr(logits), _ptr(self.ws),
                                   self.ws.numel(), _stream(stream)))

    def stage_head_rowmax(self, h, logits, rowmax, stream=None):
        """dg_stage_head_rowmax: also rowmax [T, V/64] f32 (slab maxima)."""
        _check(lib().dg_stage_head_rowmax(self.handle, h.shape[0], _ptr(h), _ptr(logits),
                                          _ptr(rowmax), _ptr(self.ws), self.ws.numel(),
                                          _stream(stream)))


# ------------------------------------------------------------------ model-free calls

def sampler_workspace(batch: int, canvas: int, device="cuda:0") -> torch.Tensor:
    n = ctypes.c_size_t()
    _check(lib().dg_sampler_workspace_bytes(batch, canvas, ctypes.byref(n)))
    return torch.empty(n.value, dtype=torch.uint8, device=device)


def sample_update(params: dict, step: int, logits, canvas, argmax, lock, stats, stop, ws,
                  stream=None):
    """dg_sample_update on device tensors: logits [B,N,V] f32, canvas/argmax [B,N] i32,
    lock [B,N] u8, stats [B,N,4] f32, stop [B] i32 (in/out)."""
    B, N, V = logits.shape
    sp = sampler_params(params)
    _check(lib().dg_sample_update(ctypes.byref(sp), int(step), B, N, V, _ptr(logits),
                                  _ptr(canvas), _ptr(argmax), _ptr(lock), _ptr(stats), _ptr(stop),
                                  _ptr(ws), ws.numel(), _stream(stream)))


def sample_update_static(params: dict, step: int, logits, canvas, argmax, lock, stats, stop,
                         stream=None):
    """dg_sample_update_static: sample_update with the library's static scratch
    (no workspace; batch * canvas <= 65536)."""
    B, N, V = logits.shape
    sp = sampler_params(params)
    _check(lib().dg_sample_update_static(ctypes.byref(sp), int(step), B, N, V, _ptr(logits),
                                         _ptr(canvas), _ptr(argmax), _ptr(lock), _ptr(stats),
                                         _ptr(stop), _stream(stream)))


def sample_update_probs(params: dict, step: int, logits, canvas, argmax, lock, stats, stop,
                        rowmax, probs, ws, blocked: bool = True, stream=None):
    """dg_sample_update_probs: sample_update, and probs (bf16 storage; blocked
    layout over B*N rows padded to 256, or row-major) from rowmax [B*N, V/64] f32."""
    B, N, V = logits.shape
    sp = sampler_params(params)
    _check(lib().dg_sample_update_probs(ctypes.byref(sp), int(step), B, N, V, _ptr(logits),
                                        _ptr(canvas), _ptr(argmax), _ptr(lock), _ptr(stats),
                                        _ptr(stop), _ptr(rowmax), 1 if blocked else 0, _ptr(probs),
                                        _ptr(ws), ws.numel(), _stream(stream)))


def corrupt(seed: int, step: int, vocab: int, rate, clean, out, stream=None):
    """dg_corrupt: clean [B, N] int32, rate [B] f32 -> out [B, N] int32."""
    B, N = clean.shape
    _check(lib().dg_corrupt(int(seed), int(step), B, N, int(vocab), _ptr(rate), _ptr(clean),
                            _ptr(out), _stream(stream)))


def xent(logits, target, loss, mean=None, stream=None):
    """dg_xent: logits [R, V] f32, target [R] int32 -> loss [R] f32, mean [1] f32."""
    R, V = logits.shape
    _check(lib().dg_xent(R, V, _ptr(logits), _ptr(target), _ptr(loss),
                         _ptr(mean) if mean is not None else None, _stream(stream)))


def argmax_rows(logits, out, stream=None):
    """dg_argmax_rows: logits [R, V] f32 -> out [R] int32 (ties to the lower index)."""
    R, V = logits.shape
    _check(lib().dg_argmax_rows(R, V, _ptr(logits), _ptr(out), _stream(stream)))


def stage_probs(logits, stats, probs, blocked: bool, stream=None):
    """dg_stage_probs: logits [T, V] f32, stats [T, 4] f32 -> probs (bf16 storage)."""
    T, V = logits.shape
    _check(lib().dg_stage_probs(T, V, 1 if blocked else 0, _ptr(logits), _ptr(stats), _ptr(probs),
                                _stream(stream)))


def quantize_fp8(src, q, scale, stream=None):
    """dg_quantize_fp8: src [..., cols] (f32 or bf16; rows % 16 == 0, cols %
    128 == 0) -> q (uint8, rows * cols bytes in the tiled layout of
    include/dg.h) and scale (f32, one per row)."""
    cols = src.shape[-1]
    rows = src.numel() // cols
    dt = DG_BF16 if src.dtype == torch.bfloat16 else DG_F32
    _check(lib().dg_quantize_fp8(_ptr(src), dt, rows, cols, _ptr(q), _ptr(scale), _stream(stream)))


def quantize_mxfp4(src, codes, scales, stream=None):
    """dg_quantize_mxfp4: src [..., cols] (f32 or bf16; rows % 16 == 0, cols %
    128 == 0) -> codes (uint8, rows * cols/2 bytes, two codes a byte) and
    scales (uint8, rows * cols/32), both in the tiled layout of include/dg.h."""
    cols = src.shape[-1]
    rows = src.numel() // cols
    dt = DG_BF16 if src.dtype == torch.bfloat16 else DG_F32
    _check(lib().dg_quantize_mxfp4(_ptr(src), dt, rows, cols, _ptr(codes), _ptr(scales),
                                   _stream(stream)))


def timer_enable(names) -> None:
    """Start the library's kernel timers for the given names (see TIMERS)."""
    mask = 0
    for n in names:
        mask |= 1 << TIMERS[n]
    _check(lib().dg_timer_enable(mask))


def timer_read(name: str):
    """(total ms, launches) recorded for a timer since timer_enable."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().dg_timer_read(TIMERS[name], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def measure_peaks(buf, stream=None):
    """(HBM read GB/s, bf16 MFMA TFLOP/s) measured by the library's probe
    kernels on a device buffer of at least 256 MiB (a calibration aid)."""
    gbs = ctypes.c_double()
    tf = ctypes.c_double()
    _check(lib().dg_measure_peaks(_ptr(buf), buf.numel() * buf.element_size(), _stream(stream),
                                  ctypes.byref(gbs), ctypes.byref(tf)))
    return gbs.value, tf.value


def canvas_init(seed: int, block_index: int, canvas, vocab: int, stream=None):
    B, N = canvas.shape
    _check(lib().dg_canvas_init(int(seed), int(block_index), B, N, int(vocab), _ptr(canvas),
                                _stream(stream)))
