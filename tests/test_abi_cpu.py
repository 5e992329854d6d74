"""The C-ABI library without a GPU: it loads, exports every declared entry point,
and its host-side argument checks return the documented status codes."""
import ctypes
import os
import re

import pytest

from gpt_pre_norm_amd import gpt2mi as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gpt2mi.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt2_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = G.load()
    names = declared_functions()
    assert set(names) == set(G.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for st in range(9):
        assert G.status_str(st)
    assert G.status_str(6).startswith("token id")


def test_workspace_size_host_logic():
    hp = G.hparams()
    small = G.workspace_size(hp, G.BF16, 1, 1)
    big = G.workspace_size(hp, G.BF16, 8, 1024)
    assert 0 < small < big
    assert G.workspace_size(hp, G.FP32, 8, 1024) > big
    assert G.workspace_size(hp, 5, 1, 1) == 0
    assert G.workspace_size(G.hparams(n_embd=770, n_head=10), G.BF16, 1, 1) == 0  # d_h = 77
    assert G.workspace_size(G.hparams(n_embd=64, n_head=4), G.BF16, 1, 1) > 0     # bf16 at d_h 16
    assert G.workspace_size(G.hparams(n_embd=768, n_head=4), G.BF16, 1, 1) == 0   # d_h 192 > 128
    assert G.workspace_size(G.hparams(n_embd=96, n_head=16), G.BF16, 1, 1) == 0   # d_h 6 not a multiple of 4
    assert G.workspace_size(G.hparams(n_embd=64, n_head=4), G.FP32, 1, 1) > 0
    assert G.workspace_size(hp, G.BF16, 0, 1) == 0


FAKE = 0x1000  # never dereferenced: every call below fails its host-side checks


def _block_weights():
    return G.BlockWeights(*([FAKE] * 12))


@pytest.mark.parametrize("case,expect", [
    ("bad_mode", 3), ("bad_heads", 2), ("null_x", 1), ("null_weight", 1), ("T_over_ctx", 4),
    ("zero_B", 2), ("small_ws", 5), ("null_ws", 1), ("misaligned_ws", 5), ("misaligned_x", 8),
    ("misaligned_weight", 8)])
def test_block_forward_argument_errors(case, expect):
    lib = G.load()
    hp = G.hparams(n_ctx=16)
    mode, B, T, x, ws, nbytes = G.BF16, 1, 4, FAKE, FAKE, 1 << 40
    w = _block_weights()
    if case == "bad_mode":
        mode = 7
    elif case == "bad_heads":
        hp = G.hparams(n_embd=768, n_head=7)
    elif case == "null_x":
        x = None
    elif case == "null_weight":
        w.fc_b = None
    elif case == "T_over_ctx":
        T = 17
    elif case == "zero_B":
        B = 0
    elif case == "small_ws":
        nbytes = 1024
    elif case == "null_ws":
        ws = None
    elif case == "misaligned_ws":
        ws = FAKE + 16  # regions are carved at 256-byte offsets from the start
    elif case == "misaligned_x":
        x = FAKE + 8    # rows are read with 16-byte vector loads
    elif case == "misaligned_weight":
        w.attn_w = FAKE + 2
    st = lib.gpt2_block_forward(ctypes.byref(hp), mode, ctypes.byref(w), x, FAKE, B, T, None, ws, nbytes,
                                None)
    assert st == expect, (st, G.STATUS.get(st))


def test_decode_and_forward_position_errors():
    lib = G.load()
    hp = G.hparams(n_ctx=1024, n_layer=2)
    blocks = (G.BlockWeights * 2)(_block_weights(), _block_weights())
    W = G.Weights(FAKE, FAKE, FAKE, FAKE, ctypes.cast(blocks, ctypes.POINTER(G.BlockWeights)))
    kv = G.KV(FAKE, 1024)
    big = 1 << 40
    # l_past + 1 must stay within n_ctx ("strictly below n_ctx")
    assert lib.gpt2_decode_step(ctypes.byref(hp), G.BF16, ctypes.byref(W), FAKE, 4, 1024, ctypes.byref(kv),
                                FAKE, FAKE, big, None) == 4
    assert lib.gpt2_decode_step(ctypes.byref(hp), G.BF16, ctypes.byref(W), FAKE, 4, -1, ctypes.byref(kv),
                                FAKE, FAKE, big, None) == 4
    small = G.KV(FAKE, 100)
    assert lib.gpt2_decode_step(ctypes.byref(hp), G.BF16, ctypes.byref(W), FAKE, 4, 100, ctypes.byref(small),
                                FAKE, FAKE, big, None) == 4
    assert lib.gpt2_forward(ctypes.byref(hp), G.BF16, ctypes.byref(W), FAKE, 2, 1025, FAKE, None, FAKE, big,
                            None) == 4
    assert lib.gpt2_forward(ctypes.byref(hp), G.BF16, ctypes.byref(W), FAKE, 2, 200, FAKE, ctypes.byref(small),
                            FAKE, big, None) == 4
    assert lib.gpt2_decode_step(ctypes.byref(hp), G.BF16, ctypes.byref(W), FAKE, 4, 5, None, FAKE, FAKE, big,
                                None) == 1
    assert lib.gpt2_forward(ctypes.byref(hp), G.BF16, ctypes.byref(W), FAKE + 1, 2, 4, FAKE, None, FAKE, big,
                            None) == 8   # ids must be 4-byte aligned
    Wm = G.Weights(FAKE + 4, FAKE, FAKE, FAKE, ctypes.cast(blocks, ctypes.POINTER(G.BlockWeights)))
    assert lib.gpt2_decode_step(ctypes.byref(hp), G.BF16, ctypes.byref(Wm), FAKE, 4, 5, ctypes.byref(kv),
                                FAKE, FAKE, big, None) == 8   # wte must be 16-byte aligned
    hp0 = G.hparams(n_vocab=0)
    assert lib.gpt2_forward(ctypes.byref(hp0), G.BF16, ctypes.byref(W), FAKE, 2, 4, FAKE, None, FAKE, big,
                            None) == 2


def test_decode_noalloc_argument_errors():
    """The no-alloc decode step checks its arguments like gpt2_decode_step and
    refuses a batch whose workspace exceeds its fixed 16 MiB array, all before
    anything touches a GPU."""
    lib = G.load()
    blocks = (G.BlockWeights * 2)(_block_weights(), _block_weights())
    W = G.Weights(FAKE, FAKE, FAKE, FAKE, ctypes.cast(blocks, ctypes.POINTER(G.BlockWeights)))
    kv = G.KV(FAKE, 1024)
    hp = G.hparams(n_ctx=1024, n_layer=2)
    call = lambda hp_, B, l_past, kv_=kv, ids=FAKE: lib.gpt2_decode_step_noalloc(
        ctypes.byref(hp_), G.BF16, ctypes.byref(W), ids, B, l_past, ctypes.byref(kv_) if kv_ else None, FAKE, None)
    assert call(hp, 4, 1024) == 4      # l_past + 1 beyond n_ctx
    assert call(hp, 4, 5, kv_=None) == 1
    assert call(hp, 0, 5) == 2
    assert call(hp, 4, 5, ids=FAKE + 2) == 8
    wide = G.hparams(n_ctx=1024, n_embd=2048, n_head=32, n_layer=2)
    assert G.workspace_size(wide, G.BF16, 64, 1) <= 16 << 20 < G.workspace_size(wide, G.BF16, 400, 1)
    assert call(wide, 400, 5) == 5     # beyond the fixed array


def test_prefill_argument_errors():
    lib = G.load()
    hp = G.hparams(n_ctx=1024, n_layer=2)
    blocks = (G.BlockWeights * 2)(_block_weights(), _block_weights())
    W = G.Weights(FAKE, FAKE, FAKE, FAKE, ctypes.cast(blocks, ctypes.POINTER(G.BlockWeights)))
    kv = G.KV(FAKE, 1024)
    small = G.KV(FAKE, 600)
    big = 1 << 40

    def call(B, T, l_past, cache, ws_bytes=big):
        return lib.gpt2_prefill(ctypes.byref(hp), G.BF16, ctypes.byref(W), FAKE, B, T, l_past,
                                ctypes.byref(cache) if cache is not None else None, FAKE, FAKE, ws_bytes, None)

    # positions l_past .. l_past + T - 1 must stay below n_ctx and the capacity
    assert call(2, 25, 1000, kv) == 4
    assert call(2, 100, 512, small) == 4
    assert call(2, 10, -1, kv) == 4
    assert call(2, 0, 10, kv) == 2
    assert call(2, 10, 10, None) == 1
    assert call(2, 10, 10, kv, ws_bytes=16) == 5
    assert call(2, 10, 10, G.KV(FAKE + 8, 1024)) == 8


def test_generate_argument_errors():
    lib = G.load()
    hp = G.hparams(n_ctx=1024, n_layer=2)
    blocks = (G.BlockWeights * 2)(_block_weights(), _block_weights())
    W = G.Weights(FAKE, FAKE, FAKE, FAKE, ctypes.cast(blocks, ctypes.POINTER(G.BlockWeights)))
    kv = G.KV(FAKE, 1024)
    small = G.KV(FAKE, 600)
    big = 1 << 40

    def call(B, l_past, n_new, cache, out=FAKE, ws_bytes=big, ws=FAKE):
        return lib.gpt2_generate_greedy(ctypes.byref(hp), G.BF16, ctypes.byref(W), FAKE, B, l_past, n_new,
                                        ctypes.byref(cache) if cache is not None else None, out, ws,
                                        ws_bytes, None)

    assert call(2, 1000, 25, kv) == 4      # positions past n_ctx
    assert call(2, 590, 20, small) == 4    # past the cache capacity
    assert call(2, -1, 5, kv) == 4
    assert call(2, 10, 0, kv) == 2
    assert call(0, 10, 5, kv) == 2
    assert call(2, 10, 5, None) == 1
    assert call(2, 10, 5, kv, out=None) == 1
    assert call(2, 10, 5, kv, ws_bytes=16) == 5
    assert call(2, 10, 5, kv, ws=FAKE + 8) == 5
    assert call(2, 10, 5, kv, out=FAKE + 2) == 8
    assert call(2, 10, 5, G.KV(FAKE + 4, 1024)) == 8
    need = G.load().gpt2_generate_workspace_size(ctypes.byref(hp), G.BF16, 2)
    assert need > G.workspace_size(hp, G.BF16, 2, 1)   # the step's regions plus logits and tokens


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback path: without the built library every call site gets an error."""
    monkeypatch.setattr(G, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        G.load(str(tmp_path / "libgpt2mi.so"))


def test_binding_refuses_host_and_strided_tensors():
    import torch
    with pytest.raises(ValueError, match="device tensor"):
        G._ptr(torch.zeros(4))
    assert G._ptr(None) is None and G._ptr(FAKE) == FAKE


def test_bench_refuses_more_than_one_gpu():
    """One GPU only: --gpus N > 1 exits with a message before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr
