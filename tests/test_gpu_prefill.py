"""Chunked prefill (gpt2_prefill): a forward over T new tokens per sequence at
positions l_past.. against the K/V cache, checked against the oracle's forward
over the whole sequence ("Full Forward Pass", How it works: the past keys and
values and the new tokens; each query sees every key up to its position)."""
import numpy as np
import pytest
import torch

from gpt_pre_norm_amd import gpt2mi as G
from gpt_pre_norm_amd import synth
from gpt_pre_norm_amd.workloads import WORKLOADS, model_inputs
from oracle import gpt2_oracle as O
from tests.gpu_helpers import (check, check_argmax, hp_of, log, new_cache, run_forward, run_prefill,
                               to_np)

pytestmark = pytest.mark.gpu


def _small_model(mode, V, n_ctx, d, h, L, seed):
    bf = mode == G.BF16
    W = synth.model_weights(V, n_ctx, d, L, seed, affine="random", bf16=bf)
    return W, G.upload_model(W, mode), hp_of(V, n_ctx, d, h, L)


@pytest.mark.parametrize("mode,V,n_ctx,d,h,L,B,chunks", [
    (G.FP32, 1001, 128, 64, 4, 2, 2, (37, 1, 50)),
    (G.BF16, 1001, 512, 128, 2, 2, 2, (37, 1, 50, 129)),   # ragged offsets, one decode-sized chunk
    (G.BF16, 509, 512, 128, 2, 3, 3, (300, 200)),          # chunks spanning several 128-query tiles
    (G.BF16, 300, 256, 64, 1, 1, 1, (64, 64, 128)),        # tile-aligned offsets
])
def test_prefill_chunks(mode, V, n_ctx, d, h, L, B, chunks):
    S = sum(chunks)
    W, Wd, hp = _small_model(mode, V, n_ctx, d, h, L, 900 + S)
    ids = synth.ids_input((B, S), V, 901 + S)
    cap = S + 5
    cache = new_cache(mode, B, L, h, cap, d // h)
    ol, opres = O.model_forward(ids, W, h)
    l_past = 0
    outs = []
    for T in chunks:
        log(f"prefill mode={mode} d={d} L={L} B={B} l_past={l_past} T={T}")
        logits, st = run_prefill(mode, hp, Wd, ids[:, l_past:l_past + T], l_past, cache, cap)
        assert st == 0
        check(f"logits [{l_past}, {l_past + T})", to_np(logits), ol[:, l_past:l_past + T], mode)
        outs.append(to_np(logits))
        l_past += T
    check("cache slots [0, S)", to_np(cache)[..., :S, :], opres, mode)
    assert not to_np(cache)[..., S:, :].any()  # slots past the sequence untouched
    check_argmax(np.concatenate(outs, 1), ol, mode)


def test_prefill_chunk_matches_forward():
    """The second half of a sequence prefilled against the cache gives bit for
    bit the logits of the uncached forward over the whole sequence: every
    product is row-wise with one reduction order, and the attention keeps a
    per-query softmax state over the same 64-key tiles of absolute positions,
    to which tiles past a query add exact zeros."""
    mode, V, n_ctx, d, h, L, B, S, T1 = G.BF16, 777, 512, 128, 2, 2, 2, 400, 222
    W, Wd, hp = _small_model(mode, V, n_ctx, d, h, L, 950)
    ids = synth.ids_input((B, S), V, 951)
    full, st = run_forward(mode, hp, Wd, ids)
    assert st == 0
    cache = new_cache(mode, B, L, h, S, d // h)
    _, st = run_prefill(mode, hp, Wd, ids[:, :T1], 0, cache, S)
    assert st == 0
    tail, st = run_prefill(mode, hp, Wd, ids[:, T1:], T1, cache, S)
    assert st == 0
    err = float(np.abs(to_np(tail) - to_np(full)[:, T1:]).max())
    log(f"  chunked vs uncached max abs diff {err:.3e}")
    assert err == 0.0


def test_prefill_gpt2s_second_half():
    """GPT-2 small at full size: the 1024-token workload prefilled in two chunks
    of 512; sequences 0 and 5 of the second chunk recomputed by the oracle,
    every logit row (1024 rows for the argmax gate), and their cache slots."""
    wl = WORKLOADS["gpt2s_fwd_b8_t1024"]
    ids, W = model_inputs(wl)
    Wd = G.upload_model(W, wl.mode)
    hp = hp_of(wl.n_vocab, wl.n_ctx, wl.d, wl.h, wl.L)
    cache = new_cache(wl.mode, wl.B, wl.L, wl.h, wl.n_ctx, wl.dh)
    log("prefill gpt2-small: chunk [0, 512)")
    _, st = run_prefill(wl.mode, hp, Wd, ids[:, :512], 0, cache, wl.n_ctx)
    assert st == 0
    log("prefill gpt2-small: chunk [512, 1024)")
    logits, st = run_prefill(wl.mode, hp, Wd, ids[:, 512:], 512, cache, wl.n_ctx)
    assert st == 0
    rows = np.arange(512, 1024)
    g_all, o_all = [], []
    for b in (0, 5):
        ol, opres = O.model_forward(ids[b:b + 1], W, wl.h, logit_rows=rows)
        g = to_np(logits[b])
        check(f"logits[{b}] ({len(rows)} rows)", g, ol, wl.mode)
        check(f"cache[{b}]", to_np(cache[b:b + 1]), opres, wl.mode)
        g_all.append(g)
        o_all.append(ol)
    check_argmax(np.concatenate(g_all), np.concatenate(o_all), wl.mode, min_rows=1000)
