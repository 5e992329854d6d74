"""Fused tied head + next-token cross-entropy (gpt2_forward_loss) against the
oracle's cross-entropy of its own logits ("Full Forward Pass", How it works:
callers take a next-token cross-entropy of the logits).

Tolerance: the loss is log-sum-exp minus one logit, and log-sum-exp moves by
at most the largest logit error, so |loss error| <= 2 x the logit tolerance:
6e-2 in bf16 mode, 2 x 1e-4 x max|logit| in fp32 mode."""
import numpy as np
import pytest
import torch

from gpt_pre_norm_amd import gpt2mi as G
from gpt_pre_norm_amd import synth
from gpt_pre_norm_amd.workloads import WORKLOADS, model_inputs
from oracle import gpt2_oracle as O
from tests.gpu_helpers import TOL_BF16_ABS, TOL_FP32_REL, hp_of, log, run_forward, to_np

pytestmark = pytest.mark.gpu


def _small_model(mode, V, n_ctx, d, h, L, seed):
    bf = mode == G.BF16
    W = synth.model_weights(V, n_ctx, d, L, seed, affine="random", bf16=bf)
    return W, G.upload_model(W, mode), hp_of(V, n_ctx, d, h, L)


def _targets(ids, V, seed):
    """Next tokens: ids shifted left, the last position a fresh draw."""
    last = synth.ids_input((ids.shape[0], 1), V, seed)
    return np.concatenate([ids[:, 1:], last], axis=1).astype(np.int32)


def run_loss(mode, hp, Wd, ids, targets):
    B, T = ids.shape
    idd = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    tgd = torch.from_numpy(np.ascontiguousarray(targets, np.int32)).cuda()
    loss = torch.empty((B, T), dtype=torch.float32, device="cuda")
    ws = G.loss_workspace(hp, mode, B, T)
    G.forward_loss(hp, mode, Wd, idd, tgd, B, T, loss, ws=ws)
    torch.cuda.synchronize()
    return loss, G.read_device_flags(ws)


def _check_loss(name, g, o, ol, mode):
    err = float(np.abs(np.asarray(g, np.float64) - o).max())
    gate = 2 * TOL_BF16_ABS if mode == G.BF16 else 2 * TOL_FP32_REL * float(np.abs(ol).max())
    log(f"  {name}: max abs err {err:.3e} (gate {gate:.2e}), mean loss {float(np.mean(o)):.4f}")
    assert err <= gate, (name, err)


@pytest.mark.parametrize("mode,V,n_ctx,d,h,L,B,T", [
    (G.FP32, 1001, 64, 64, 4, 2, 2, 37),      # full-logits path
    (G.BF16, 1001, 256, 128, 2, 2, 3, 20),    # M = 60: full-logits path
    (G.BF16, 1001, 256, 128, 2, 2, 2, 150),   # M = 300: fused head, ragged last column tile
    (G.BF16, 512, 256, 64, 1, 1, 2, 96),      # V a multiple of the column tile
])
def test_loss_small(mode, V, n_ctx, d, h, L, B, T):
    W, Wd, hp = _small_model(mode, V, n_ctx, d, h, L, 1300 + T)
    ids = synth.ids_input((B, T), V, 1301 + T)
    tg = _targets(ids, V, 1302 + T)
    log(f"loss mode={mode} V={V} d={d} L={L} B={B} T={T}")
    loss, st = run_loss(mode, hp, Wd, ids, tg)
    assert st == 0
    ol, _ = O.model_forward(ids, W, h)
    _check_loss("loss", to_np(loss), O.next_token_loss(ol, tg), ol, mode)


def test_loss_equals_logits_path():
    """The fused head's loss equals the cross-entropy of gpt2_forward's own
    logits up to fp32 summation order (same products, same accumulators)."""
    mode, V, n_ctx, d, h, L, B, T = G.BF16, 5003, 256, 128, 2, 2, 2, 200
    W, Wd, hp = _small_model(mode, V, n_ctx, d, h, L, 1400)
    ids = synth.ids_input((B, T), V, 1401)
    tg = _targets(ids, V, 1402)
    loss, st = run_loss(mode, hp, Wd, ids, tg)
    assert st == 0
    logits, st = run_forward(mode, hp, Wd, ids)
    assert st == 0
    ref = O.next_token_loss(to_np(logits), tg)
    err = float(np.abs(to_np(loss) - ref).max())
    log(f"  fused vs logits-path loss max abs diff {err:.3e}")
    assert err <= 1e-4


def test_loss_bad_target():
    mode, V = G.BF16, 700
    W, Wd, hp = _small_model(mode, V, 256, 64, 1, 1, 1500)
    ids = synth.ids_input((2, 100), V, 1501)
    tg = _targets(ids, V, 1502)
    tg[1, 7] = V
    loss, st = run_loss(mode, hp, Wd, ids, tg)
    assert st == 6  # GPT2_E_TOKEN
    l = to_np(loss)
    assert np.isnan(l[1, 7]) and np.isfinite(np.delete(l.reshape(-1), 107)).all()


def test_loss_gpt2s_full():
    """GPT-2 small forward workload (B=8, T=1024, V=50257) through the fused
    head; sequences 0 and 5 recomputed by the oracle on 96 sampled positions."""
    wl = WORKLOADS["gpt2s_fwd_b8_t1024"]
    ids, W = model_inputs(wl)
    tg = _targets(ids, wl.n_vocab, wl.seed + 99)
    Wd = G.upload_model(W, wl.mode)
    hp = hp_of(wl.n_vocab, wl.n_ctx, wl.d, wl.h, wl.L)
    log("loss gpt2-small full size")
    loss, st = run_loss(wl.mode, hp, Wd, ids, tg)
    assert st == 0
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 511, 1023], rng.integers(0, 1024, 93)]))
    for b in (0, 5):
        ol, _ = O.model_forward(ids[b:b + 1], W, wl.h, logit_rows=rows)
        _check_loss(f"loss[{b}] ({len(rows)} rows)", to_np(loss[b])[rows], O.next_token_loss(ol, tg[b, rows]),
                    ol, wl.mode)
