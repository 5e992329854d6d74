"""Seeded synthetic inputs shared by the HIP path's callers and the oracle's tests.

This module holds no part of the decoder's arithmetic: it only draws numbers.
Everything is counter-based, so any slice of any tensor can be regenerated on
its own (element ``i`` of a stream depends only on ``(seed, stream, i)``).

Generator definition
--------------------
* word(seed, stream, i) = mix64(key(seed, stream) + (i + 1) * 0x9E3779B97F4A7C15)
  where mix64 is the SplitMix64 output function (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014):
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31.
  key(seed, stream) = mix64(mix64(seed) ^ (stream * 0xD1B54A32D192ED03)).
* uniform(i) = ((word >> 11) + 0.5) * 2**-53, in the open interval (0, 1).
* normal: Box-Muller on the pair (uniform(2p), uniform(2p + 1)); element 2p takes
  r*cos(2*pi*u2) and element 2p + 1 takes r*sin(2*pi*u2), r = sqrt(-2 ln u1).
* token ids: (word >> 32) * V >> 32 (multiply-shift; bias below V / 2**32).

Rounding to bfloat16 is round-to-nearest-even on the fp32 bit pattern.
"""
from __future__ import annotations

import ctypes
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_NATIVE = None


def _native():
    """The C fill routines (libgpt2synth.so, same definition), or None if not built."""
    global _NATIVE
    if _NATIVE is None:
        path = os.path.join(_HERE, "libgpt2synth.so")
        if not os.path.exists(path):
            return None
        lib = ctypes.CDLL(path)
        u64, vp = ctypes.c_uint64, ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, ctypes.c_double, ctypes.c_int, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, ctypes.c_double, vp]
        lib.synth_token_ids.argtypes = [u64, u64, u64, ctypes.c_uint32, vp]
        lib.synth_stream_key.argtypes = [u64, u64]
        lib.synth_stream_key.restype = u64
        _NATIVE = lib
    return _NATIVE

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_STREAM_MUL = 0xD1B54A32D192ED03
_MASK64 = (1 << 64) - 1
_CHUNK = 1 << 22


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & _MASK64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & _MASK64
    z ^= z >> 31
    return z


def stream_key(seed: int, stream: int) -> int:
    return _mix64_int(_mix64_int(seed) ^ ((stream * _STREAM_MUL) & _MASK64))


def _mix64(z: np.ndarray) -> np.ndarray:
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def words(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """64-bit words ``start .. start+count-1`` of one stream."""
    key = np.uint64(stream_key(seed, stream))
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = key + i * _GOLDEN
        return _mix64(z)


def _uniform(w: np.ndarray) -> np.ndarray:
    return ((w >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def _normal_range(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Normal draws for elements [start, start+count) of a stream (fp64)."""
    p0 = start // 2
    p1 = (start + count + 1) // 2
    w = words(seed, stream, 2 * p0, 2 * (p1 - p0))
    u1 = _uniform(w[0::2])
    u2 = _uniform(w[1::2])
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * math.pi * u2
    out = np.empty(2 * (p1 - p0), dtype=np.float64)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    off = start - 2 * p0
    return out[off:off + count]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(shape, std: float, seed: int, stream: int, start: int = 0,
           *, bf16: bool = False, native: bool = True) -> np.ndarray:
    """fp32 array of N(0, std) draws (computed in fp64, rounded once to fp32;
    then to bf16 when ``bf16``)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32)
    lib = _native() if native else None
    if lib is not None:
        lib.synth_normal_f32(seed, stream, start, n, float(std), int(bf16), out.ctypes.data)
        return out.reshape(shape)

    def fill(lo):
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = (_normal_range(seed, stream, start + lo, hi - lo) * std).astype(np.float32)

    starts = range(0, n, _CHUNK)
    if n > _CHUNK:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, starts))
    else:
        for lo in starts:
            fill(lo)
    out = out.reshape(shape)
    return round_bf16(out) if bf16 else out


def normal_bf16_bits(shape, std: float, seed: int, stream: int, start: int = 0) -> np.ndarray:
    """The same draws as ``normal(..., bf16=True)``, as uint16 bf16 bit patterns."""
    n = int(np.prod(shape, dtype=np.int64))
    lib = _native()
    if lib is None:
        return to_bf16_bits(normal((n,), std, seed, stream, start)).reshape(shape)
    out = np.empty(n, dtype=np.uint16)
    lib.synth_normal_bf16(seed, stream, start, n, float(std), out.ctypes.data)
    return out.reshape(shape)


def token_ids(shape, n_vocab: int, seed: int, stream: int, *, native: bool = True) -> np.ndarray:
    n = int(np.prod(shape, dtype=np.int64))
    lib = _native() if native else None
    if lib is not None:
        out = np.empty(n, dtype=np.int32)
        lib.synth_token_ids(seed, stream, n, n_vocab, out.ctypes.data)
        return out.reshape(shape)
    w = words(seed, stream, 0, n)
    ids = ((w >> np.uint64(32)) * np.uint64(n_vocab)) >> np.uint64(32)
    return ids.astype(np.int32).reshape(shape)


# ---------------------------------------------------------------- bfloat16

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. No NaN handling needed here."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16, returned as fp32."""
    return bf16_bits_to_f32(to_bf16_bits(x))


# ---------------------------------------------------------------- model inputs

BLOCK_KEYS = ("ln1_g", "ln1_b", "attn_w", "attn_b", "proj_w", "proj_b",
              "ln2_g", "ln2_b", "fc_w", "fc_b", "fc2_w", "fc2_b")

# stream ids: one per tensor kind, layer folded in
_S_X, _S_IDS, _S_WTE, _S_WPE, _S_PAST, _S_LNF = 1, 2, 3, 4, 5, 6
_S_BLOCK0 = 100


def block_weights(d: int, seed: int, layer: int = 0, *, std: float = 0.02,
                  resid_scale: float = 1.0, affine: str = "default",
                  bf16: bool = False) -> dict:
    """One block's parameters, linear weights stored [out, in].

    affine="default": LN gains 1, LN biases 0, linear biases 0 (the workloads' recipe).
    affine="random": gains 1 + N(0, 0.1), LN biases N(0, 0.1), linear biases N(0, 0.02),
    so that every bias and affine term is exercised by parity tests.
    """
    base = _S_BLOCK0 + 16 * layer
    shapes = {"attn_w": (3 * d, d), "proj_w": (d, d), "fc_w": (4 * d, d), "fc2_w": (d, 4 * d)}
    scale = {"attn_w": std, "proj_w": std * resid_scale, "fc_w": std, "fc2_w": std * resid_scale}
    w = {}
    for j, k in enumerate(("attn_w", "proj_w", "fc_w", "fc2_w")):
        w[k] = normal(shapes[k], scale[k], seed, base + j, bf16=bf16)
    vec = {"ln1_g": d, "ln1_b": d, "attn_b": 3 * d, "proj_b": d,
           "ln2_g": d, "ln2_b": d, "fc_b": 4 * d, "fc2_b": d}
    for j, k in enumerate(("ln1_g", "ln1_b", "attn_b", "proj_b", "ln2_g", "ln2_b", "fc_b", "fc2_b")):
        n = vec[k]
        if affine == "random":
            if k.endswith("_g"):
                w[k] = (1.0 + normal((n,), 0.1, seed, base + 4 + j)).astype(np.float32)
            elif k.startswith("ln"):
                w[k] = normal((n,), 0.1, seed, base + 4 + j)
            else:
                w[k] = normal((n,), 0.02, seed, base + 4 + j)
        else:
            w[k] = (np.ones if k.endswith("_g") else np.zeros)((n,), dtype=np.float32)
    if bf16:  # the matrices were drawn already rounded; round the vectors
        w = {k: (v if k.endswith("_w") else round_bf16(v)) for k, v in w.items()}
    return {k: w[k] for k in BLOCK_KEYS}


def model_weights(n_vocab: int, n_ctx: int, d: int, n_layer: int, seed: int, *,
                  affine: str = "default", bf16: bool = False,
                  resid_scale: float | None = None) -> dict:
    """wte ~ N(0, 0.02), wpe ~ N(0, 0.01), blocks as block_weights with residual
    projections scaled by 1/sqrt(2 * n_layer) unless resid_scale is given."""
    if resid_scale is None:
        resid_scale = 1.0 / math.sqrt(2 * n_layer)
    wte = normal((n_vocab, d), 0.02, seed, _S_WTE, bf16=bf16)
    wpe = normal((n_ctx, d), 0.01, seed, _S_WPE, bf16=bf16)
    if affine == "random":
        lnf_g = (1.0 + normal((d,), 0.1, seed, _S_LNF)).astype(np.float32)
        lnf_b = normal((d,), 0.1, seed, _S_LNF + 1000)
    else:
        lnf_g = np.ones((d,), np.float32)
        lnf_b = np.zeros((d,), np.float32)
    W = {"wte": wte, "wpe": wpe, "lnf_g": lnf_g, "lnf_b": lnf_b}
    if bf16:  # wte and wpe were drawn already rounded
        W = {k: (v if k in ("wte", "wpe") else round_bf16(v)) for k, v in W.items()}
    W["blocks"] = [block_weights(d, seed, l, resid_scale=resid_scale, affine=affine, bf16=bf16)
                   for l in range(n_layer)]
    return W


def hidden_input(shape, seed: int, *, bf16: bool = False) -> np.ndarray:
    return normal(shape, 1.0, seed, _S_X, bf16=bf16)


def ids_input(shape, n_vocab: int, seed: int) -> np.ndarray:
    return token_ids(shape, n_vocab, seed, _S_IDS)


def past_normal(shape, seed: int, *, start: int = 0, bf16: bool = False) -> np.ndarray:
    """N(0,1) draws for a KV cache region; ``start`` offsets into the flat stream."""
    return normal(shape, 1.0, seed, _S_PAST, start=start, bf16=bf16)


def past_bf16_bits(shape, seed: int, *, start: int = 0) -> np.ndarray:
    """The same KV-cache draws as bf16 bit patterns (uint16)."""
    return normal_bf16_bits(shape, 1.0, seed, _S_PAST, start=start)
