"""Greedy generation (gpt2_generate_greedy): n decode steps on the device,
each feeding back the argmax of its logits.  Every chosen token is checked to
be a greedy choice under the oracle's logits for the sequence the GPU built
("Full Forward Pass", How it works: a generation loop over cached decode
steps), and the loop against step-by-step decoding through the C ABI."""
import numpy as np
import pytest
import torch

from gpt_pre_norm_amd import gpt2mi as G
from gpt_pre_norm_amd import synth
from gpt_pre_norm_amd.workloads import WORKLOADS, model_inputs, past_for_sequence
from oracle import gpt2_oracle as O
from tests.gpu_helpers import (TOL_BF16_ABS, check, hp_of, log, new_cache, run_decode, run_prefill, to_np)

pytestmark = pytest.mark.gpu


def _small_model(mode, V, n_ctx, d, h, L, seed):
    bf = mode == G.BF16
    W = synth.model_weights(V, n_ctx, d, L, seed, affine="random", bf16=bf)
    return W, G.upload_model(W, mode), hp_of(V, n_ctx, d, h, L)


def _generate(mode, hp, Wd, first_ids, l_past, n_new, cache, cap):
    B = first_ids.shape[0]
    idd = torch.from_numpy(np.ascontiguousarray(first_ids, np.int32)).cuda()
    out = torch.full((B, n_new), -1, dtype=torch.int32, device="cuda")
    ws = G.generate_workspace(hp, mode, B)
    G.generate_greedy(hp, mode, Wd, idd, B, l_past, n_new, cache, cap, out, ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _assert_greedy(tokens, logits, mode, what):
    """tokens [n], oracle logits [n, V]: each token's logit within the
    tolerance of the row maximum (exactly the maximum up to fp32 error in fp32 mode)."""
    o = np.asarray(logits, np.float64)
    mx = o.max(-1)
    got = o[np.arange(len(tokens)), tokens]
    tol = TOL_BF16_ABS if mode == G.BF16 else 1e-4 * np.abs(o).max()
    gap = mx - got
    log(f"  {what}: {len(tokens)} tokens, max gap to the oracle's best logit {gap.max():.3e} (tol {tol:.1e}); "
        f"{(gap == 0).mean():.3f} exact argmax")
    assert (gap <= tol).all(), gap


@pytest.mark.parametrize("mode,V,n_ctx,d,h,L,B,T0,n_new", [
    (G.FP32, 301, 128, 64, 4, 2, 2, 9, 12),
    (G.BF16, 1001, 256, 128, 2, 2, 3, 40, 24),
    # from an empty cache (the first token at position 0) to the last position
    (G.BF16, 501, 16, 128, 2, 2, 2, 1, 16),
    # B = 66 > 64: full bf16 logits, then the row argmax kernel
    (G.BF16, 211, 128, 128, 2, 2, 66, 20, 6),
])
def test_generate_greedy_valid(mode, V, n_ctx, d, h, L, B, T0, n_new):
    W, Wd, hp = _small_model(mode, V, n_ctx, d, h, L, 1100 + T0)
    prompt = synth.ids_input((B, T0), V, 1101 + T0)
    cap = min(T0 + n_new + 3, n_ctx)
    cache = new_cache(mode, B, L, h, cap, d // h)
    if T0 > 1:
        _, st = run_prefill(mode, hp, Wd, prompt[:, :T0 - 1], 0, cache, cap)
        assert st == 0
    log(f"generate mode={mode} d={d} L={L} B={B} from position {T0 - 1}, {n_new} tokens")
    gen = _generate(mode, hp, Wd, prompt[:, T0 - 1], T0 - 1, n_new, cache, cap)
    assert ((gen >= 0) & (gen < V)).all()
    seq = np.concatenate([prompt, gen[:, :-1]], axis=1)  # every token that was fed
    ol, opres = O.model_forward(seq, W, h)
    for b in range(B):
        _assert_greedy(gen[b], ol[b, T0 - 1:], mode, f"sequence {b}")
    S = seq.shape[1]
    check("cache slots [0, S)", to_np(cache)[..., :S, :], opres, mode)
    assert not to_np(cache)[..., S:, :].any()


def test_generate_matches_decode_steps():
    """The device loop equals host-driven decode steps with torch's argmax
    (first maximal index), token for token and in the cache."""
    mode, V, n_ctx, d, h, L, B, T0, n_new = G.BF16, 997, 256, 128, 2, 2, 4, 17, 20
    W, Wd, hp = _small_model(mode, V, n_ctx, d, h, L, 1200)
    prompt = synth.ids_input((B, T0), V, 1201)
    cap = T0 + n_new
    caches = [new_cache(mode, B, L, h, cap, d // h) for _ in range(2)]
    for c in caches:
        _, st = run_prefill(mode, hp, Wd, prompt[:, :T0 - 1], 0, c, cap)
        assert st == 0
    gen = _generate(mode, hp, Wd, prompt[:, T0 - 1], T0 - 1, n_new, caches[0], cap)
    tok = prompt[:, T0 - 1]
    ref = []
    for i in range(n_new):
        logits = run_decode(mode, hp, Wd, tok, T0 - 1 + i, caches[1], cap)
        tok = logits[:, 0].argmax(-1).int().cpu().numpy()
        ref.append(tok)
    ref = np.stack(ref, 1)
    assert np.array_equal(gen, ref)
    assert torch.equal(caches[0], caches[1])


@pytest.mark.parametrize("case", ["all_zero", "two_rows"])
def test_generate_ties_lowest_index(case):
    """Tied logits: the device choice is the lowest column among equal maxima,
    across tiles of the head product.  all_zero: wte = 0, so every logit is
    exactly 0 and every chosen token is 0.  two_rows: wte = 0 except rows
    300 and 9000 equal to v and rows 200 and 8000 equal to -v, so whatever the
    sign of a position's logit for v, the maximum is a tie between two columns
    in different tiles (300 or 200 must win); the loop must also match
    host-driven steps with torch's argmax."""
    mode, V, n_ctx, d, h, L, B, T0, n_new = G.BF16, 10007, 64, 128, 2, 1, 3, 5, 6
    W = synth.model_weights(V, n_ctx, d, L, 1300, affine="random", bf16=True)
    W["wte"][:] = 0.0
    if case == "two_rows":
        v = synth.normal((d,), 0.5, 1301, 0, bf16=True)
        W["wte"][300] = v
        W["wte"][9000] = v
        W["wte"][200] = -v
        W["wte"][8000] = -v
    Wd, hp = G.upload_model(W, mode), hp_of(V, n_ctx, d, h, L)
    prompt = synth.ids_input((B, T0), V, 1302)
    cap = T0 + n_new
    caches = [new_cache(mode, B, L, h, cap, d // h) for _ in range(2)]
    for c in caches:
        _, st = run_prefill(mode, hp, Wd, prompt[:, :T0 - 1], 0, c, cap)
        assert st == 0
    gen = _generate(mode, hp, Wd, prompt[:, T0 - 1], T0 - 1, n_new, caches[0], cap)
    if case == "all_zero":
        assert (gen == 0).all(), gen
        return
    tok = prompt[:, T0 - 1]
    ref = []
    for i in range(n_new):
        logits = run_decode(mode, hp, Wd, tok, T0 - 1 + i, caches[1], cap)
        tok = logits[:, 0].argmax(-1).int().cpu().numpy()
        ref.append(tok)
    ref = np.stack(ref, 1)
    log(f"  two tied pairs: chosen {np.unique(gen)}")
    assert np.isin(gen, (200, 300)).all(), gen
    assert np.array_equal(gen, ref), (gen, ref)


def test_generate_gpt2s_full():
    """GPT-2 small, 64 sequences with a random past of 1000 positions, 16
    greedy tokens; sequences 0 and 37 replayed by the oracle's cached decode."""
    wl = WORKLOADS["gpt2s_decode_b64_p1023"]
    ids, W = model_inputs(wl)
    first = ids[:, 0]
    Wd = G.upload_model(W, wl.mode)
    hp = hp_of(wl.n_vocab, wl.n_ctx, wl.d, wl.h, wl.L)
    l_past, n_new, cap = 1000, 16, wl.n_ctx
    log("generate gpt2-small: placing the past")
    cache = new_cache(wl.mode, wl.B, wl.L, wl.h, cap, wl.dh)
    per_seq = wl.L * 2 * wl.h * wl.l_past * wl.dh
    bits = synth.past_bf16_bits((wl.B * per_seq,), wl.seed)
    past = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    cache[..., :l_past, :] = past.view(wl.B, wl.L, 2, wl.h, wl.l_past, wl.dh)[..., :l_past, :]
    del past, bits
    gen = _generate(wl.mode, hp, Wd, first, l_past, n_new, cache, cap)
    for b in (0, 37):
        pb = past_for_sequence(wl, b)[None][..., :l_past, :]
        tok = first[b:b + 1]
        logits = []
        for i in range(n_new):
            ol, pres = O.decode_step(tok, W, wl.h, past=pb)
            logits.append(ol[0, 0])
            pb = np.concatenate([pb, pres], axis=4)
            tok = gen[b:b + 1, i]
        _assert_greedy(gen[b], np.stack(logits), wl.mode, f"sequence {b}")
