"""gpt2_decode_step_noalloc, the decode step whose workspace is the library's
own device array (for callers that cannot allocate), against gpt2_decode_step
with a caller's workspace: the same logits and cache slot, on two calls in a
row, the second with a smaller batch."""
import numpy as np
import pytest
import torch

from gpt_pre_norm_amd import gpt2mi as G
from gpt_pre_norm_amd import synth
from tests.gpu_helpers import hp_of, log, new_cache, run_forward, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.load()


def _decode_both(mode, hp, Wd, ids, l_past, cache, cap):
    """(logits, new K/V) of the workspace step and of the no-alloc step, each
    on its own copy of the cache."""
    B = ids.shape[0]
    idd = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    outs = []
    for noalloc in (False, True):
        c = cache.clone()
        logits = torch.full((B, 1, hp.n_vocab), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            G.decode_step_noalloc(hp, mode, Wd, idd, B, l_past, c, cap, logits)
        else:
            ws = G.workspace(hp, mode, B, 1)
            G.decode_step(hp, mode, Wd, idd, B, l_past, c, cap, logits, ws=ws)
        torch.cuda.synchronize()
        outs.append((to_np(logits), to_np(c[..., l_past, :])))
    return outs


@pytest.mark.parametrize("mode", [G.FP32, G.BF16])
def test_noalloc_matches_workspace_step(mode):
    V, n_ctx, d, h, L = 701, 128, 128, 2, 2
    bf = mode == G.BF16
    W = synth.model_weights(V, n_ctx, d, L, 1300, affine="random", bf16=bf)
    Wd, hp = G.upload_model(W, mode), hp_of(V, n_ctx, d, h, L)
    for B, T in ((6, 40), (3, 25)):  # the second call smaller than the first
        ids = synth.ids_input((B, T), V, 1301 + B)
        cache = new_cache(mode, B, L, h, n_ctx, d // h)
        _, st = run_forward(mode, hp, Wd, ids[:, :T - 1], cache=cache, capacity=n_ctx)
        assert st == 0
        (lw, kvw), (ln, kvn) = _decode_both(mode, hp, Wd, ids[:, T - 1], T - 1, cache, n_ctx)
        assert np.isfinite(ln).all()
        # the same kernels in the same order on the same inputs: the same bits
        # (the decode step adds its K-range partials in a fixed order)
        log(f"  mode={mode} B={B}: logits identical {np.array_equal(lw, ln)}, "
            f"max abs diff {float(np.abs(lw - ln).max()):.3e}")
        assert np.array_equal(lw, ln)
        assert np.array_equal(kvw, kvn)


def test_noalloc_rejects_oversized_batch():
    V, d, h, L = 301, 2048, 32, 1
    W = synth.model_weights(V, 16, d, L, 1310, bf16=True)
    Wd, hp = G.upload_model(W, G.BF16), hp_of(V, 16, d, h, L)
    B = 400  # about 18 MB of workspace at n_embd 2048, over the 16 MiB array
    ids = torch.zeros(B, dtype=torch.int32, device="cuda")
    cache = new_cache(G.BF16, B, L, h, 16, d // h)
    logits = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
    with pytest.raises(G.Gpt2Error) as e:
        G.decode_step_noalloc(hp, G.BF16, Wd, ids, B, 3, cache, 16, logits)
    assert e.value.status == 5  # GPT2_E_WORKSPACE


def test_noalloc_graph_replays_match_eager():
    """The no-alloc step is meant for code under HIP graph capture: captured
    once and replayed several times, with eager work between the replays,
    every replay gives the eager no-alloc step's bits."""
    V, n_ctx, d, h, L, B, T = 701, 128, 256, 4, 2, 16, 30
    W = synth.model_weights(V, n_ctx, d, L, 1320, affine="random", bf16=True)
    Wd, hp = G.upload_model(W, G.BF16), hp_of(V, n_ctx, d, h, L)
    ids = synth.ids_input((B, T), V, 1321)
    cache = new_cache(G.BF16, B, L, h, n_ctx, d // h)
    _, st = run_forward(G.BF16, hp, Wd, ids[:, :T - 1], cache=cache, capacity=n_ctx)
    assert st == 0
    idd = torch.from_numpy(np.ascontiguousarray(ids[:, T - 1], np.int32)).cuda()
    logits = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
    G.decode_step_noalloc(hp, G.BF16, Wd, idd, B, T - 1, cache, n_ctx, logits)
    torch.cuda.synchronize()
    eager_logits, eager_kv = logits.clone(), cache[..., T - 1, :].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.decode_step_noalloc(hp, G.BF16, Wd, idd, B, T - 1, cache, n_ctx, logits)
    for rep in range(4):
        logits.fill_(float("nan"))
        cache[..., T - 1, :] = 0
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(logits, eager_logits) and torch.equal(cache[..., T - 1, :], eager_kv)
        log(f"  no-alloc replay {rep}: identical to the eager step {same}")
        assert same
        # eager work between replays, on the same device array: a smaller
        # no-alloc step of other sequences
        c2 = new_cache(G.BF16, 3, L, h, n_ctx, d // h)
        l2 = torch.empty((3, 1, V), dtype=torch.float32, device="cuda")
        G.decode_step_noalloc(hp, G.BF16, Wd, idd[:3], 3, 5, c2, n_ctx, l2)
        torch.cuda.synchronize()
