"""ctypes front end of the C sampler oracle (``oracle/sampler.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.

The C file fixes the sampler's binary32 arithmetic (the pages leave it open);
this module only marshals numpy arrays.  ``build()`` compiles it with gcc.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sampler.c")
_LIB = os.path.join(_HERE, "liboracle_sampler.so")
_lib = None

LOCK_MAXPROB = 0
LOCK_CUMENT = 1


def build(force: bool = True) -> str:
    """Compile sampler.c into liboracle_sampler.so next to it (gcc, -O2, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
            "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        f32, i32, u64 = ctypes.c_float, ctypes.c_int32, ctypes.c_uint64
        P = ctypes.c_void_p
        L.ora_exp.restype = f32
        L.ora_exp.argtypes = [f32]
        L.ora_log.restype = f32
        L.ora_log.argtypes = [f32]
        L.ora_philox4x64.restype = None
        L.ora_philox4x64.argtypes = [P, P, P]
        L.ora_uniform.restype = f32
        L.ora_uniform.argtypes = [u64]
        L.ora_uniform_token.restype = i32
        L.ora_uniform_token.argtypes = [u64, i32]
        L.ora_row_stats.restype = None
        L.ora_row_stats.argtypes = [P, ctypes.c_int, P, P]
        L.ora_draw.restype = i32
        L.ora_draw.argtypes = [P, ctypes.c_int, f32, f32, f32, f32]
        L.ora_inv_temperature.restype = f32
        L.ora_inv_temperature.argtypes = [f32, f32, ctypes.c_int, ctypes.c_int]
        L.ora_canvas_init.restype = None
        L.ora_canvas_init.argtypes = [u64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, P]
        L.ora_sample_update.restype = None
        L.ora_sample_update.argtypes = [ctypes.c_int, f32, f32, f32, f32, ctypes.c_int,
                                        ctypes.c_int, u64, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, P, P, P, P, P, P]
        L.ora_topk_row.restype = i32
        L.ora_topk_row.argtypes = [P, ctypes.c_int, ctypes.c_int, f32, f32, P, P, P]
        L.ora_sample_update_topk.restype = None
        L.ora_sample_update_topk.argtypes = [ctypes.c_int, f32, f32, f32, f32, ctypes.c_int,
                                             ctypes.c_int, u64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P,
                                             P, P, P]
        L.ora_corrupt.restype = None
        L.ora_corrupt.argtypes = [u64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  P, P, P]
        L.ora_xent.restype = f32
        L.ora_xent.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def exp32(x: float) -> np.float32:
    return np.float32(lib().ora_exp(float(x)))


def log32(x: float) -> np.float32:
    return np.float32(lib().ora_log(float(x)))


def philox4x64(counter, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint64))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64))
    out = np.zeros(4, dtype=np.uint64)
    lib().ora_philox4x64(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(word: int) -> np.float32:
    return np.float32(lib().ora_uniform(int(word)))


def uniform_token(word: int, V: int) -> int:
    return int(lib().ora_uniform_token(int(word), int(V)))


def row_stats(row: np.ndarray):
    """(m, S, H, pmax), argmax of one float32 logit row."""
    row = np.ascontiguousarray(row, dtype=np.float32)
    out = np.zeros(4, dtype=np.float32)
    am = np.zeros(1, dtype=np.int32)
    lib().ora_row_stats(_ptr(row), row.size, _ptr(out), _ptr(am))
    return out, int(am[0])


def draw(row: np.ndarray, inv_t: float, u1: float, u2: float, u3: float) -> int:
    row = np.ascontiguousarray(row, dtype=np.float32)
    return int(lib().ora_draw(_ptr(row), row.size, float(np.float32(inv_t)), float(u1),
                              float(u2), float(u3)))


def inv_temperature(T0: float, T1: float, step: int, max_steps: int) -> np.float32:
    return np.float32(lib().ora_inv_temperature(float(T0), float(T1), int(step), int(max_steps)))


def canvas_init(seed: int, block: int, B: int, N: int, V: int) -> np.ndarray:
    out = np.zeros((B, N), dtype=np.int32)
    lib().ora_canvas_init(int(seed), int(block), int(B), int(N), int(V), _ptr(out))
    return out


def corrupt(seed: int, step: int, V: int, rate: np.ndarray, clean: np.ndarray) -> np.ndarray:
    """Multinomial corruption of clean [B, N] int32 at per-canvas rates [B]
    (float32) over a vocabulary of V: the training-side forward's input, as
    sampler.c defines it."""
    clean = np.ascontiguousarray(clean, dtype=np.int32)
    rate = np.ascontiguousarray(rate, dtype=np.float32)
    B, N = clean.shape
    out = np.zeros_like(clean)
    lib().ora_corrupt(int(seed), int(step), B, N, int(V), _ptr(rate), _ptr(clean), _ptr(out))
    return out


def xent(logits: np.ndarray, target: np.ndarray):
    """Cross-entropy of float32 logit rows [R, V] at target [R]:
    (per-row losses float32 [R], mean float32)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    R, V = lg.shape
    t = np.ascontiguousarray(target, dtype=np.int32).reshape(-1)
    assert t.size == R and (t >= 0).all() and (t < V).all()
    loss = np.zeros(R, dtype=np.float32)
    mean = np.float32(lib().ora_xent(_ptr(lg), R, V, _ptr(t), _ptr(loss)))
    return loss, mean


def topk_row(row: np.ndarray, K: int, inv_t: float, u: float):
    """Top-k truncated statistics of one float32 row: (stats [m, S, H, pmax],
    candidates idx [K], self-conditioning weights p [K], drawn token)."""
    row = np.ascontiguousarray(row, dtype=np.float32)
    Ke = min(K, row.size)
    out = np.zeros(4, dtype=np.float32)
    idx = np.zeros(Ke, dtype=np.int32)
    p = np.zeros(Ke, dtype=np.float32)
    y = int(lib().ora_topk_row(_ptr(row), row.size, int(K), float(np.float32(inv_t)),
                               float(np.float32(u)), _ptr(out), _ptr(idx), _ptr(p)))
    return out, idx, p, y


def sample_update(params: dict, step: int, logits: np.ndarray, canvas: np.ndarray,
                  argmax: np.ndarray, stop: np.ndarray):
    """One sampler update.  logits [B,N,V] float32; canvas/argmax [B,N] int32 and
    stop [B] int32 are updated in place; returns (lock [B,N] uint8, stats [B,N,4]).
    params["top_k"] > 0 selects top-k truncation."""
    B, N, V = logits.shape
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    assert canvas.dtype == np.int32 and argmax.dtype == np.int32 and stop.dtype == np.int32
    lock = np.zeros((B, N), dtype=np.uint8)
    stats = np.zeros((B, N, 4), dtype=np.float32)
    common = (int(params["lock_rule"]), float(params["lock_theta"]), float(params["temp_start"]),
              float(params["temp_end"]), float(params["stop_tau"]), int(params["require_stable"]),
              int(params["max_steps"]), int(params["seed"]), int(step))
    K = int(params.get("top_k", 0))
    if K > 0:
        lib().ora_sample_update_topk(*common, K, B, N, V, _ptr(logits), _ptr(canvas),
                                     _ptr(argmax), _ptr(lock), _ptr(stats), _ptr(stop))
    else:
        lib().ora_sample_update(*common, B, N, V, _ptr(logits), _ptr(canvas), _ptr(argmax),
                                _ptr(lock), _ptr(stats), _ptr(stop))
    return lock, stats
