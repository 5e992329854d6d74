"""The decode step captured into a HIP graph and replayed, as the benchmark
times it, against the same step launched eagerly.

Each replay rewrites cache slot l_past with the same K/V ("Full Forward
Pass", How it works: the cached step appends the new token's K/V and attends
over slots 0..l_past), so replays are idempotent. The graph is replayed
several times with eager work between the replays, and every replay must give
the eager step's bits (the decode step adds its K-range partials in a fixed
order). The logits are also checked against the oracle."""
import numpy as np
import pytest
import torch

from gpt_pre_norm_amd import gpt2mi as G
from gpt_pre_norm_amd import synth
from oracle import gpt2_oracle as O
from tests.gpu_helpers import check, hp_of, log, new_cache, run_forward, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.load()


@pytest.mark.parametrize("mode", [G.FP32, G.BF16])
def test_decode_graph_replays_match_eager(mode):
    V, n_ctx, d, h, L, B, T = 1001, 128, 768, 12, 2, 64, 40
    bf = mode == G.BF16
    W = synth.model_weights(V, n_ctx, d, L, 1400, affine="random", bf16=bf)
    Wd, hp = G.upload_model(W, mode), hp_of(V, n_ctx, d, h, L)
    ids = synth.ids_input((B, T), V, 1401)
    cache = new_cache(mode, B, L, h, n_ctx, d // h)
    _, st = run_forward(mode, hp, Wd, ids[:, :T - 1], cache=cache, capacity=n_ctx)
    assert st == 0
    idd = torch.from_numpy(np.ascontiguousarray(ids[:, T - 1], np.int32)).cuda()
    logits = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
    ws = G.workspace(hp, mode, B, 1)

    G.decode_step(hp, mode, Wd, idd, B, T - 1, cache, n_ctx, logits, ws=ws)
    torch.cuda.synchronize()
    eager_logits, eager_kv = logits.clone(), cache[..., T - 1, :].clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.decode_step(hp, mode, Wd, idd, B, T - 1, cache, n_ctx, logits, ws=ws)
    for rep in range(4):
        logits.fill_(float("nan"))
        cache[..., T - 1, :] = 0
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(logits, eager_logits) and torch.equal(cache[..., T - 1, :], eager_kv)
        log(f"  mode={mode} replay {rep}: identical to the eager step {same}")
        assert same
        # eager work between replays: the uncached forward over the same tokens
        _, st = run_forward(mode, hp, Wd, ids[:, :T - 1], cache=cache, capacity=n_ctx)
        assert st == 0
    ol, _ = O.model_forward(ids, W, h, logit_rows=np.arange(B) * T + T - 1)
    check("logits", to_np(eager_logits)[:, 0], ol, mode)
