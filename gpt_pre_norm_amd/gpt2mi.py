"""ctypes binding of libgpt2mi.so (include/gpt2mi.h).

Argument marshalling only: every step of the decoder runs in the HIP library.
torch supplies device memory and the current stream; torch is imported before
the library is loaded so that both bind to the same HIP runtime.  Loading fails
loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2mi.so")

FP32, BF16 = 0, 1
STATUS = {0: "GPT2_OK", 1: "GPT2_E_NULL", 2: "GPT2_E_SHAPE", 3: "GPT2_E_DTYPE",
          4: "GPT2_E_POSITION", 5: "GPT2_E_WORKSPACE", 6: "GPT2_E_TOKEN", 7: "GPT2_E_HIP",
          8: "GPT2_E_ALIGN"}
EXPORTS = ("gpt2_workspace_size", "gpt2_block_forward", "gpt2_forward", "gpt2_prefill", "gpt2_decode_step",
           "gpt2_decode_step_noalloc",
           "gpt2_generate_workspace_size", "gpt2_generate_greedy", "gpt2_loss_workspace_size",
           "gpt2_forward_loss", "gpt2_read_device_flags",
           "gpt2_timing_begin", "gpt2_timing_end", "gpt2_status_str")
BLOCK_KEYS = ("ln1_g", "ln1_b", "attn_w", "attn_b", "proj_w", "proj_b",
              "ln2_g", "ln2_b", "fc_w", "fc_b", "fc2_w", "fc2_b")


class Gpt2Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class HParams(ctypes.Structure):
    _fields_ = [("n_vocab", ctypes.c_int32), ("n_ctx", ctypes.c_int32), ("n_embd", ctypes.c_int32),
                ("n_head", ctypes.c_int32), ("n_layer", ctypes.c_int32), ("eps", ctypes.c_float)]


class BlockWeights(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in BLOCK_KEYS]


class Weights(ctypes.Structure):
    _fields_ = [("wte", ctypes.c_void_p), ("wpe", ctypes.c_void_p), ("lnf_g", ctypes.c_void_p),
                ("lnf_b", ctypes.c_void_p), ("blocks", ctypes.POINTER(BlockWeights))]


class KV(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("capacity", ctypes.c_int32)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libgpt2mi.so once; raises if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m gpt_pre_norm_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    hp_p = ctypes.POINTER(HParams)
    lib.gpt2_workspace_size.argtypes = [hp_p, ctypes.c_int, i32, i32]
    lib.gpt2_workspace_size.restype = sz
    lib.gpt2_block_forward.argtypes = [hp_p, ctypes.c_int, ctypes.POINTER(BlockWeights), vp, vp, i32, i32,
                                       vp, vp, sz, vp]
    lib.gpt2_forward.argtypes = [hp_p, ctypes.c_int, ctypes.POINTER(Weights), vp, i32, i32, vp,
                                 ctypes.POINTER(KV), vp, sz, vp]
    lib.gpt2_prefill.argtypes = [hp_p, ctypes.c_int, ctypes.POINTER(Weights), vp, i32, i32, i32,
                                 ctypes.POINTER(KV), vp, vp, sz, vp]
    lib.gpt2_decode_step.argtypes = [hp_p, ctypes.c_int, ctypes.POINTER(Weights), vp, i32, i32,
                                     ctypes.POINTER(KV), vp, vp, sz, vp]
    lib.gpt2_decode_step_noalloc.argtypes = [hp_p, ctypes.c_int, ctypes.POINTER(Weights), vp, i32, i32,
                                             ctypes.POINTER(KV), vp, vp]
    lib.gpt2_generate_workspace_size.argtypes = [hp_p, ctypes.c_int, i32]
    lib.gpt2_generate_workspace_size.restype = sz
    lib.gpt2_generate_greedy.argtypes = [hp_p, ctypes.c_int, ctypes.POINTER(Weights), vp, i32, i32, i32,
                                         ctypes.POINTER(KV), vp, vp, sz, vp]
    lib.gpt2_loss_workspace_size.argtypes = [hp_p, ctypes.c_int, i32, i32]
    lib.gpt2_loss_workspace_size.restype = sz
    lib.gpt2_forward_loss.argtypes = [hp_p, ctypes.c_int, ctypes.POINTER(Weights), vp, vp, i32, i32, vp,
                                      ctypes.POINTER(KV), vp, sz, vp]
    lib.gpt2_read_device_flags.argtypes = [vp, vp]
    lib.gpt2_timing_begin.argtypes = []
    lib.gpt2_timing_begin.restype = ctypes.c_int
    lib.gpt2_timing_end.argtypes = [ctypes.POINTER(KernelTime), i32]
    lib.gpt2_timing_end.restype = i32
    lib.gpt2_status_str.argtypes = [ctypes.c_int]
    lib.gpt2_status_str.restype = ctypes.c_char_p
    for f in ("gpt2_block_forward", "gpt2_forward", "gpt2_prefill", "gpt2_decode_step", "gpt2_decode_step_noalloc",
              "gpt2_generate_greedy",
              "gpt2_forward_loss", "gpt2_read_device_flags"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------------- marshalling helpers

def hparams(n_vocab=50257, n_ctx=1024, n_embd=768, n_head=12, n_layer=12, eps=1e-5) -> HParams:
    return HParams(n_vocab, n_ctx, n_embd, n_head, n_layer, eps)


def _ptr(t) -> int | None:
    """Device address of a tensor (None and raw integer addresses pass through).
    The C ABI takes dense row-major device buffers: a host tensor or a strided
    view is refused here rather than read as if it were dense."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(st: int, what: str):
    if st != 0:
        raise Gpt2Error(st, what)


def to_device(a: np.ndarray, mode: int, device="cuda") -> torch.Tensor:
    """Host array -> device tensor of the mode dtype (bf16 by round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device, dtype=torch.bfloat16 if mode == BF16 else torch.float32)


def block_struct(w: dict) -> BlockWeights:
    return BlockWeights(*[_ptr(w[k]) for k in BLOCK_KEYS])


class ModelWeights:
    """Device weights plus the ctypes structs that point at them (keeps both alive)."""

    def __init__(self, W: dict):
        self.tensors = W
        self.blocks = (BlockWeights * len(W["blocks"]))(*[block_struct(b) for b in W["blocks"]])
        self.struct = Weights(_ptr(W["wte"]), _ptr(W["wpe"]), _ptr(W["lnf_g"]), _ptr(W["lnf_b"]),
                              ctypes.cast(self.blocks, ctypes.POINTER(BlockWeights)))


def upload_block(w: dict, mode: int, device="cuda") -> dict:
    return {k: to_device(w[k], mode, device) for k in BLOCK_KEYS}


def upload_model(W: dict, mode: int, device="cuda") -> ModelWeights:
    dev = {k: to_device(W[k], mode, device) for k in ("wte", "wpe", "lnf_g", "lnf_b")}
    dev["blocks"] = [upload_block(b, mode, device) for b in W["blocks"]]
    return ModelWeights(dev)


# ---------------------------------------------------------------- entry points

def workspace_size(hp: HParams, mode: int, B: int, T: int) -> int:
    return int(load().gpt2_workspace_size(ctypes.byref(hp), mode, B, T))


def workspace(hp: HParams, mode: int, B: int, T: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of the required size (uint8 tensor)."""
    n = workspace_size(hp, mode, B, T)
    if n == 0:
        raise Gpt2Error(2, "gpt2_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def block_forward(hp: HParams, mode: int, w, x, y, B: int, T: int, present=None, ws=None,
                  stream=None, ws_bytes=None):
    ws_bytes = ws.numel() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    ws_ = w if isinstance(w, BlockWeights) else block_struct(w)
    _check(load().gpt2_block_forward(ctypes.byref(hp), mode, ctypes.byref(ws_), _ptr(x), _ptr(y), B, T,
                                     _ptr(present), _ptr(ws), ws_bytes, _stream(stream)),
           "gpt2_block_forward")


def forward(hp: HParams, mode: int, W: ModelWeights, ids, B: int, T: int, logits, present=None,
            capacity: int | None = None, ws=None, stream=None, ws_bytes=None):
    ws_bytes = ws.numel() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    kv = None
    if present is not None:
        kv = KV(_ptr(present), capacity if capacity is not None else T)
    _check(load().gpt2_forward(ctypes.byref(hp), mode, ctypes.byref(W.struct), _ptr(ids), B, T,
                               _ptr(logits), ctypes.byref(kv) if kv is not None else None, _ptr(ws),
                               ws_bytes, _stream(stream)), "gpt2_forward")


def prefill(hp: HParams, mode: int, W: ModelWeights, ids, B: int, T: int, l_past: int, cache, capacity: int,
            logits, ws=None, stream=None, ws_bytes=None):
    ws_bytes = ws.numel() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    kv = KV(_ptr(cache), capacity)
    _check(load().gpt2_prefill(ctypes.byref(hp), mode, ctypes.byref(W.struct), _ptr(ids), B, T, l_past,
                               ctypes.byref(kv), _ptr(logits), _ptr(ws), ws_bytes, _stream(stream)),
           "gpt2_prefill")


def decode_step(hp: HParams, mode: int, W: ModelWeights, ids, B: int, l_past: int, cache, capacity: int,
                logits, ws=None, stream=None, ws_bytes=None):
    ws_bytes = ws.numel() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    kv = KV(_ptr(cache), capacity)
    _check(load().gpt2_decode_step(ctypes.byref(hp), mode, ctypes.byref(W.struct), _ptr(ids), B, l_past,
                                   ctypes.byref(kv), _ptr(logits), _ptr(ws), ws_bytes, _stream(stream)),
           "gpt2_decode_step")


def decode_step_noalloc(hp: HParams, mode: int, W: ModelWeights, ids, B: int, l_past: int, cache, capacity: int,
                        logits, stream=None):
    kv = KV(_ptr(cache), capacity)
    _check(load().gpt2_decode_step_noalloc(ctypes.byref(hp), mode, ctypes.byref(W.struct), _ptr(ids), B, l_past,
                                           ctypes.byref(kv), _ptr(logits), _stream(stream)),
           "gpt2_decode_step_noalloc")


def generate_workspace(hp: HParams, mode: int, B: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for generate_greedy (uint8 tensor)."""
    n = int(load().gpt2_generate_workspace_size(ctypes.byref(hp), mode, B))
    if n == 0:
        raise Gpt2Error(2, "gpt2_generate_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def generate_greedy(hp: HParams, mode: int, W: ModelWeights, ids, B: int, l_past: int, n_new: int, cache,
                    capacity: int, out, ws=None, stream=None, ws_bytes=None):
    ws_bytes = ws.numel() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    kv = KV(_ptr(cache), capacity)
    _check(load().gpt2_generate_greedy(ctypes.byref(hp), mode, ctypes.byref(W.struct), _ptr(ids), B, l_past,
                                       n_new, ctypes.byref(kv), _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
           "gpt2_generate_greedy")


def loss_workspace(hp: HParams, mode: int, B: int, T: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for forward_loss (uint8 tensor)."""
    n = int(load().gpt2_loss_workspace_size(ctypes.byref(hp), mode, B, T))
    if n == 0:
        raise Gpt2Error(2, "gpt2_loss_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def forward_loss(hp: HParams, mode: int, W: ModelWeights, ids, targets, B: int, T: int, loss, present=None,
                 capacity: int | None = None, ws=None, stream=None, ws_bytes=None):
    ws_bytes = ws.numel() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    kv = None
    if present is not None:
        kv = KV(_ptr(present), capacity if capacity is not None else T)
    _check(load().gpt2_forward_loss(ctypes.byref(hp), mode, ctypes.byref(W.struct), _ptr(ids), _ptr(targets), B, T,
                                    _ptr(loss), ctypes.byref(kv) if kv is not None else None, _ptr(ws),
                                    ws_bytes, _stream(stream)), "gpt2_forward_loss")


def read_device_flags(ws, stream=None) -> int:
    """Returns the status (0 or GPT2_E_TOKEN) and clears the flags."""
    return int(load().gpt2_read_device_flags(_ptr(ws), _stream(stream)))


def timing_begin() -> None:
    _check(load().gpt2_timing_begin(), "gpt2_timing_begin")


def timing_end() -> dict:
    """{kernel name: (launches, total ms)} for the launches since timing_begin()."""
    buf = (KernelTime * 32)()
    n = load().gpt2_timing_end(buf, 32)
    if n < 0:
        raise Gpt2Error(7, "gpt2_timing_end")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n, 32))}


def status_str(st: int) -> str:
    return load().gpt2_status_str(st).decode()
