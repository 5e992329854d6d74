#!/usr/bin/env python3
"""Throughput of the GPT-2 pre-norm decoder on one MI355X, through the C ABI.

One step = one uncached bf16 forward of GPT-2 small over B=8 sequences of
T=1024 synthetic tokens (embedding, 12 pre-norm blocks, ln_f, tied head with
fp32 logits [8, 1024, 50257]).  `value` is tokens/s of that forward.  The same
run also times the cached decode step (64 sequences, one new token each at
position 1023 against a random past) and reports it under "decode".

Per-kernel durations come from HIP events the library records around each
launch (gpt2_timing_begin/end) on the launch stream, in a pass after the
timed region; the roofline object prices the dominant kernel's algorithmic
work against MI355X's published peaks.  The CPU oracle is timed on a bounded
sample of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps K2]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s & %bf16 MFMA peak, GPT-2-small fwd B8 T1024; decode tok/s, %HBM"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the chunked-prefill, loss and generation measurements")
    return ap.parse_args()


def traffic_for(phase: str, kernel: str):
    """HBM-side bytes per launch of a kernel kind, measured with rocprofv3
    FETCH_SIZE / WRITE_SIZE counters (scaled by a calibration copy) and kept in
    profiles/traffic.json with a hash of the kernel sources; None when absent or
    when the sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        from gpt_pre_norm_amd.profiling import sources_sha
        rec = json.load(open(path))
    except (OSError, ValueError, ImportError):
        return None
    if rec.get("source_sha") != sources_sha():
        return None
    k = rec.get(phase, {}).get(kernel)
    return None if k is None else round(k["bytes_per_launch"])


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(it would shard the batch, one replica per GPU); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from gpt_pre_norm_amd import gpt2mi as G
    from gpt_pre_norm_amd import roofline as R
    from gpt_pre_norm_amd import synth
    from gpt_pre_norm_amd.workloads import WORKLOADS, model_inputs

    G.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------ forward workload
    wl = WORKLOADS["gpt2s_fwd_b8_t1024"]
    log(f"[bench] generating {wl.name}")
    ids_np, W = model_inputs(wl)
    Wd = G.upload_model(W, G.BF16)
    hp = G.hparams(n_vocab=wl.n_vocab, n_ctx=wl.n_ctx, n_embd=wl.d, n_head=wl.h, n_layer=wl.L)
    ids = torch.from_numpy(ids_np).to(dev)
    logits = torch.empty((wl.B, wl.T, wl.n_vocab), dtype=torch.float32, device=dev)
    ws = G.workspace(hp, G.BF16, wl.B, wl.T)

    def fwd():
        G.forward(hp, G.BF16, Wd, ids, wl.B, wl.T, logits, ws=ws, stream=stream)

    log(f"[bench] forward warmup {args.warmup}")
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    if G.read_device_flags(ws) != 0:
        raise SystemExit("token flag raised")
    warm_rows = logits[:, :64].clone()  # a warm-up step's output, for the determinism check
    log(f"[bench] forward timed steps {args.steps}")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        fwd()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = max(wall * 1e3, gpu_ms) / args.steps
    # the forward is deterministic (no atomics at B*T > 64 rows): the timed
    # steps' logits equal the first step's; the host keeps sequences 0..3 for
    # the comparison with the oracle in the CPU-baseline leg
    gpu_seqs = None if args.no_cpu_baseline else logits[:4].cpu().numpy()
    deterministic = bool(torch.equal(warm_rows, logits[:, :64]))
    del warm_rows
    tokens_per_s = wl.tokens / (ms_per_step / 1e3)
    flops = R.model_flops(wl.B, wl.T, wl.d, wl.h, wl.L, wl.n_vocab)
    log(f"[bench] forward {ms_per_step:.3f} ms/step, {tokens_per_s:.4g} tok/s, "
        f"{flops / (ms_per_step / 1e3) / 1e12:.1f} TFLOP/s")

    # per-kernel pass (events around each launch)
    G.timing_begin()
    for _ in range(args.steps):
        fwd()
    kt = G.timing_end()
    work = dict(B=wl.B, T=wl.T, d=wl.d, h=wl.h, V=wl.n_vocab)
    kernels = {}
    for name, (n, tot) in sorted(kt.items(), key=lambda kv: -kv[1][1]):
        f, b = R.kernel_work(name, **work)
        avg_s = tot / n / 1e3
        kernels[name] = {"launches_per_step": n / args.steps, "avg_us": round(avg_s * 1e6, 2),
                         "share": round(tot / sum(v[1] for v in kt.values()), 4),
                         "tflops": round(f / avg_s / 1e12, 1), "gbps": round(b / avg_s / 1e9, 1)}
        log(f"[bench]   {name:22s} {n // args.steps:4d}/step avg {avg_s * 1e6:9.2f} us "
            f"{f / avg_s / 1e12:8.1f} TFLOP/s {b / avg_s / 1e9:8.1f} GB/s")
    dom = max(kt.items(), key=lambda kv: kv[1][1])[0]
    f, b = R.kernel_work(dom, **work)
    n, tot = kt[dom]
    avg_s = tot / n / 1e3
    bound = R.bound_of(f, b)
    if bound == "mfma":
        achieved, peak, unit = f / avg_s / 1e12, R.PEAK_BF16_FLOPS / 1e12, "TFLOP/s"
    else:
        achieved, peak, unit = b / avg_s / 1e9, R.PEAK_HBM_BYTES / 1e9, "GB/s"
    roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic_for("forward", dom),
                "work_per_launch": f if bound == "mfma" else b, "avg_launch_us": round(avg_s * 1e6, 2)}

    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GPT-2 small uncached forward, bf16 (fp32 accumulate, fp32 residual "
                               "stream, fp32 logits), B=8 T=1024, V=50257 d=768 h=12 L=12",
                   "batch": wl.B, "seq_len": wl.T, "parallelism": "none (1 GPU)"},
        "tflops": round(flops / (ms_per_step / 1e3) / 1e12, 1),
        "mfma_peak_frac": round(flops / (ms_per_step / 1e3) / R.PEAK_BF16_FLOPS, 4),
        "roofline": roofline,
        "kernels": kernels,
    }
    del logits, ws
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ chunked prefill, loss
    if not args.no_extras:
        result["prefill_chunk"] = bench_prefill_chunk(args, G, R, wl, Wd, hp, ids, stream, dev)
        result["forward_loss"] = bench_forward_loss(args, G, R, wl, Wd, hp, ids, stream, dev)
        result["block"] = bench_block(args, G, R, WORKLOADS["block_gpt2s_bf16"], stream, dev)
        result["block_d64_fp32"] = bench_block_tiny(args, G, WORKLOADS["block_d64_fp32"], dev)
        result["layernorm_hbm"] = bench_layernorm_hbm(args, G, R, WORKLOADS["block_gpt2s_bf16"], stream, dev)
        for key, name in (("forward_l24_d1024", "gpt2_l24_d1024_fwd_b4_t1024"),
                          ("forward_l36_d1280", "gpt2_l36_d1280_fwd_b4_t1024"),
                          ("forward_l48_d1600", "gpt2_l48_d1600_fwd_b4_t1024")):
            result[key] = bench_wide_forward(args, G, R, WORKLOADS[name], model_inputs, stream, dev)

    # ------------------------------------------------------------ decode workload
    if not args.no_decode:
        result["decode"] = bench_decode(args, G, R, synth, WORKLOADS["gpt2s_decode_b64_p1023"], Wd, hp,
                                        stream, dev)

    # ------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(wl, ids_np, W, gpu_seqs)
        if result["parity"] is not None:
            result["parity"]["warmup_equals_timed_bitwise"] = deterministic

    print(json.dumps(result), flush=True)


def _timed_loop(fn, n):
    import torch
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(n):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    return max((time.perf_counter() - t0) * 1e3, ev0.elapsed_time(ev1)) / n


def bench_prefill_chunk(args, G, R, wl, Wd, hp, ids, stream, dev):
    """The forward workload's second half, 512 new tokens per sequence at
    positions 512..1023, prefilled against the cache that the first half
    filled (rerunning it rewrites the same slots with the same values)."""
    import torch

    half = wl.T // 2
    cache = torch.zeros((wl.B, wl.L, 2, wl.h, wl.n_ctx, wl.dh), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((wl.B, half, wl.n_vocab), dtype=torch.float32, device=dev)
    ws = G.workspace(hp, G.BF16, wl.B, half)
    first, second = ids[:, :half].contiguous(), ids[:, half:].contiguous()
    G.prefill(hp, G.BF16, Wd, first, wl.B, half, 0, cache, wl.n_ctx, logits, ws=ws, stream=stream)

    def chunk():
        G.prefill(hp, G.BF16, Wd, second, wl.B, half, half, cache, wl.n_ctx, logits, ws=ws, stream=stream)

    for _ in range(max(1, args.warmup)):
        chunk()
    ms = _timed_loop(chunk, args.steps)
    flops = R.model_flops(wl.B, half, wl.d, wl.h, wl.L, wl.n_vocab) + 4.0 * wl.d * wl.B * half * half * wl.L
    log(f"[bench] prefill chunk (512 tokens at 512..1023, B={wl.B}) {ms:.3f} ms, "
        f"{wl.B * half / (ms / 1e3):.4g} tok/s, {flops / (ms / 1e3) / 1e12:.1f} TFLOP/s")
    del cache, logits, ws
    torch.cuda.empty_cache()
    return {"value": round(wl.B * half / (ms / 1e3), 1), "unit": "tokens/s", "ms": round(ms, 4),
            "tflops": round(flops / (ms / 1e3) / 1e12, 1),
            "workload": "GPT-2 small, B=8, 512 new tokens per sequence at positions 512..1023 "
                        "against a cache holding positions 0..511 (gpt2_prefill)"}


def bench_forward_loss(args, G, R, wl, Wd, hp, ids, stream, dev):
    """The forward workload with the fused head + next-token cross-entropy
    (targets = ids shifted by one); no logits are written."""
    import torch

    targets = torch.cat([ids[:, 1:], ids[:, :1]], dim=1).contiguous()
    loss = torch.empty((wl.B, wl.T), dtype=torch.float32, device=dev)
    ws = G.loss_workspace(hp, G.BF16, wl.B, wl.T)

    def run():
        G.forward_loss(hp, G.BF16, Wd, ids, targets, wl.B, wl.T, loss, ws=ws, stream=stream)

    for _ in range(max(1, args.warmup)):
        run()
    ms = _timed_loop(run, args.steps)
    G.timing_begin()
    run()
    kt = G.timing_end()
    head_us = kt["gemm_lm_head"][1] * 1e3 / kt["gemm_lm_head"][0]
    loss_us = kt["loss"][1] * 1e3 / kt["loss"][0]
    flops = R.model_flops(wl.B, wl.T, wl.d, wl.h, wl.L, wl.n_vocab)
    log(f"[bench] forward + loss {ms:.3f} ms/step, {wl.tokens / (ms / 1e3):.4g} tok/s; fused head {head_us:.1f} us, "
        f"loss rows {loss_us:.1f} us")
    del loss, ws
    torch.cuda.empty_cache()
    return {"value": round(wl.tokens / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
            "tflops": round(flops / (ms / 1e3) / 1e12, 1), "head_us": round(head_us, 2),
            "loss_rows_us": round(loss_us, 2),
            "workload": "GPT-2 small forward B=8 T=1024 with the tied head fused into the next-token "
                        "cross-entropy (gpt2_forward_loss); per-position losses, no logits written"}


def bench_block(args, G, R, wl, stream, dev):
    """One GPT-2-small block at full size through gpt2_block_forward (bf16,
    B=8, T=1024, present written)."""
    import torch
    from gpt_pre_norm_amd.workloads import block_inputs

    x_np, w = block_inputs(wl)
    hp = G.hparams(n_vocab=1, n_ctx=wl.n_ctx, n_embd=wl.d, n_head=wl.h, n_layer=1)
    wd = G.upload_block(w, G.BF16)
    x = G.to_device(x_np, G.BF16)
    y = torch.empty_like(x)
    pres = torch.empty((wl.B, 2, wl.h, wl.T, wl.dh), dtype=torch.bfloat16, device=dev)
    ws = G.workspace(hp, G.BF16, wl.B, wl.T)

    def run():
        G.block_forward(hp, G.BF16, wd, x, y, wl.B, wl.T, present=pres, ws=ws, stream=stream)

    for _ in range(max(1, args.warmup)):
        run()
    ms = _timed_loop(run, 5 * args.steps)
    flops = R.model_flops(wl.B, wl.T, wl.d, wl.h, 1, 0)
    log(f"[bench] block B={wl.B} T={wl.T} d={wl.d}: {ms * 1e3:.1f} us, {wl.tokens / (ms / 1e3):.4g} tok/s, "
        f"{flops / (ms / 1e3) / 1e12:.1f} TFLOP/s")
    del x, y, pres, ws, wd
    torch.cuda.empty_cache()
    return {"value": round(wl.tokens / (ms / 1e3), 1), "unit": "tokens/s", "us_per_call": round(ms * 1e3, 2),
            "tflops": round(flops / (ms / 1e3) / 1e12, 1),
            "mfma_peak_frac": round(flops / (ms / 1e3) / R.PEAK_BF16_FLOPS, 4),
            "workload": "one GPT-2-small block (gpt2_block_forward), bf16, B=8 T=1024 d=768 h=12, "
                        "present written"}


def bench_wide_forward(args, G, R, wl, model_inputs, stream, dev):
    """A deeper published depth (L=24 d=1024, L=36 d=1280 or L=48 d=1600;
    B=4, T=1024), uncached forward with fp32 logits."""
    import torch

    log(f"[bench] generating {wl.name}")
    ids_np, W = model_inputs(wl)
    Wd = G.upload_model(W, G.BF16)
    del W
    hp = G.hparams(n_vocab=wl.n_vocab, n_ctx=wl.n_ctx, n_embd=wl.d, n_head=wl.h, n_layer=wl.L)
    ids = torch.from_numpy(ids_np).to(dev)
    logits = torch.empty((wl.B, wl.T, wl.n_vocab), dtype=torch.float32, device=dev)
    ws = G.workspace(hp, G.BF16, wl.B, wl.T)

    def run():
        G.forward(hp, G.BF16, Wd, ids, wl.B, wl.T, logits, ws=ws, stream=stream)

    for _ in range(max(1, args.warmup)):
        run()
    ms = _timed_loop(run, max(3, args.steps // 2))
    flops = R.model_flops(wl.B, wl.T, wl.d, wl.h, wl.L, wl.n_vocab)
    log(f"[bench] forward L={wl.L} d={wl.d} B={wl.B} T={wl.T}: {ms:.3f} ms/step, "
        f"{wl.tokens / (ms / 1e3):.4g} tok/s, {flops / (ms / 1e3) / 1e12:.1f} TFLOP/s")
    del logits, ws, Wd
    torch.cuda.empty_cache()
    return {"value": round(wl.tokens / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
            "tflops": round(flops / (ms / 1e3) / 1e12, 1),
            "mfma_peak_frac": round(flops / (ms / 1e3) / R.PEAK_BF16_FLOPS, 4),
            "workload": f"L={wl.L} d={wl.d} h={wl.h} uncached forward, bf16, B={wl.B} T={wl.T}, V={wl.n_vocab}, "
                        "fp32 logits"}


def bench_block_tiny(args, G, wl, dev):
    """Latency of the small fp32 block (d=64, 4 heads, x [2, 8, 64]) through
    gpt2_block_forward: launched eagerly and replayed from a HIP graph."""
    import torch
    from gpt_pre_norm_amd.workloads import block_inputs

    x_np, w = block_inputs(wl)
    hp = G.hparams(n_vocab=1, n_ctx=wl.n_ctx, n_embd=wl.d, n_head=wl.h, n_layer=1)
    wd = G.upload_block(w, G.FP32)
    x = G.to_device(x_np, G.FP32)
    y = torch.empty_like(x)
    ws = G.workspace(hp, G.FP32, wl.B, wl.T)
    side = torch.cuda.Stream()

    def run():
        G.block_forward(hp, G.FP32, wd, x, y, wl.B, wl.T, ws=ws)

    with torch.cuda.stream(side):
        for _ in range(5):
            run()
        torch.cuda.synchronize()
        eager_ms = _timed_loop(run, 200)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            run()
    graph.replay()
    torch.cuda.synchronize()
    graph_ms = _timed_loop(graph.replay, 200)
    log(f"[bench] block d=64 fp32 B={wl.B} T={wl.T}: {eager_ms * 1e3:.1f} us eager, {graph_ms * 1e3:.1f} us graph")
    return {"us_per_call_eager": round(eager_ms * 1e3, 2), "us_per_call_graph": round(graph_ms * 1e3, 2),
            "workload": "one fp32 block (gpt2_block_forward), d=64 h=4 FFN 256, x [2, 8, 64]: latency"}


def bench_layernorm_hbm(args, G, R, wl, stream, dev):
    """LayerNorm bandwidth on a working set far above the 256 MB last-level
    cache: one GPT-2-small block over 262144 rows (B=256, T=1024), whose LN1
    reads 403 MB of bf16 x and LN2 805 MB of the fp32 stream, each writing a
    403 MB bf16 LN output; both timed with the library's per-launch events."""
    import torch
    from gpt_pre_norm_amd import synth

    B, T, d, h = 256, 1024, wl.d, wl.h
    w = synth.block_weights(d, wl.seed, 0, resid_scale=wl.resid_scale, bf16=True)
    hp = G.hparams(n_vocab=1, n_ctx=T, n_embd=d, n_head=h, n_layer=1)
    wd = G.upload_block(w, G.BF16)
    x = torch.randn((B, T, d), device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    ws = G.workspace(hp, G.BF16, B, T)

    def run():
        G.block_forward(hp, G.BF16, wd, x, y, B, T, ws=ws, stream=stream)

    run()
    torch.cuda.synchronize()
    G.timing_begin()
    for _ in range(3):
        run()
    kt = G.timing_end()
    n, tot = kt["layernorm"]
    M = B * T
    byt = M * d * (2 + 2) + M * d * (4 + 2)  # LN1: bf16 in/out; LN2: fp32 in, bf16 out
    gbps = byt * (n / 2) / (tot / 1e3) / 1e9
    log(f"[bench] layernorm over {M} rows x {d}: {tot / n * 1e3:.1f} us per launch, {gbps:.0f} GB/s")
    del x, y, ws, wd
    torch.cuda.empty_cache()
    return {"gbps": round(gbps, 1), "hbm_frac": round(gbps * 1e9 / R.PEAK_HBM_BYTES, 4),
            "avg_launch_us": round(tot / n * 1e3, 2), "bytes_per_pair": byt,
            "workload": f"LN1 + LN2 of one GPT-2-small block over {M} rows of {d} (B=256, T=1024): "
                        "1.21 GB and 0.81 GB per launch, beyond the last-level cache"}


def bench_decode(args, G, R, synth, wl, Wd, hp, stream, dev):
    import numpy as np
    import torch

    log(f"[bench] generating {wl.name} past ({wl.B}x{wl.L}x2x{wl.h}x{wl.l_past}x{wl.dh} bf16)")
    cap = wl.n_ctx
    cache = torch.empty((wl.B, wl.L, 2, wl.h, cap, wl.dh), dtype=torch.bfloat16, device=dev)
    per_seq = wl.L * 2 * wl.h * wl.l_past * wl.dh
    chunk = 8
    for b0 in range(0, wl.B, chunk):
        bits = synth.past_bf16_bits((chunk * per_seq,), wl.seed, start=b0 * per_seq)
        part = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        cache[b0:b0 + chunk, ..., :wl.l_past, :] = part.view(chunk, wl.L, 2, wl.h, wl.l_past, wl.dh)
    del part
    ids = torch.from_numpy(synth.ids_input((wl.B, 1), wl.n_vocab, wl.seed)[:, 0].copy()).to(dev)
    logits = torch.empty((wl.B, 1, wl.n_vocab), dtype=torch.float32, device=dev)
    ws = G.workspace(hp, G.BF16, wl.B, 1)

    def step():
        # rewrites slot l_past with the same K/V each time: steps are idempotent
        G.decode_step(hp, G.BF16, Wd, ids, wl.B, wl.l_past, cache, cap, logits, ws=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    timed_loop = _timed_loop

    ms_eager = timed_loop(step, args.decode_steps)
    # the same step captured once into a HIP graph and replayed (the ~100
    # launches of a step are what the graph saves; the kernels are identical)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.decode_step(hp, G.BF16, Wd, ids, wl.B, wl.l_past, cache, cap, logits, ws=ws)
    graph.replay()
    torch.cuda.synchronize()
    ms = timed_loop(graph.replay, args.decode_steps)
    byt = R.decode_bytes(wl.B, wl.d, wl.h, wl.L, wl.n_vocab, wl.l_past)
    log(f"[bench] decode eager {ms_eager * 1e3:.1f} us/step; graph {ms * 1e3:.1f} us/step, "
        f"{wl.B / (ms / 1e3):.4g} tok/s, {byt / (ms / 1e3) / 1e9:.0f} GB/s algorithmic")
    G.timing_begin()
    for _ in range(args.decode_steps):
        step()
    kt = G.timing_end()
    work = dict(B=wl.B, T=1, d=wl.d, h=wl.h, V=wl.n_vocab, l_past=wl.l_past)
    kernels = {}
    for name, (n, tot) in sorted(kt.items(), key=lambda kv: -kv[1][1]):
        f, b = R.kernel_work(name, **work)
        avg_s = tot / n / 1e3
        kernels[name] = {"launches_per_step": n / args.decode_steps, "avg_us": round(avg_s * 1e6, 2),
                         "share": round(tot / sum(v[1] for v in kt.values()), 4),
                         "gbps": round(b / avg_s / 1e9, 1)}
        log(f"[bench]   {name:22s} {n // args.decode_steps:4d}/step avg {avg_s * 1e6:9.2f} us "
            f"{b / avg_s / 1e9:8.1f} GB/s")
    dom = max(kt.items(), key=lambda kv: kv[1][1])[0]
    f, b = R.kernel_work(dom, **work)
    n, tot = kt[dom]
    avg_s = tot / n / 1e3
    ach = b / avg_s / 1e9

    result = {
        "value": round(wl.B / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "steps": args.decode_steps, "launch": "hip graph replay of one decode step",
        "ms_per_step_eager": round(ms_eager, 4),
        "workload": "GPT-2 small cached decode, bf16, B=64, one new token at position 1023, "
                    "past [64,12,2,12,1023,64] ~ N(0,1)",
        "hbm_frac_whole_step": round(byt / (ms / 1e3) / R.PEAK_HBM_BYTES, 4),
        "algorithmic_bytes_per_step": byt,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": R.PEAK_HBM_BYTES / 1e9,
                     "unit": "GB/s", "frac": round(ach * 1e9 / R.PEAK_HBM_BYTES, 4),
                     "traffic": traffic_for("decode", dom), "work_per_launch": b, "avg_launch_us": round(avg_s * 1e6, 2)},
        "kernels": kernels,
    }
    if args.no_extras:
        return result

    # greedy generation: 32 tokens from position 991 on the same cache (the
    # loop rewrites slots 991..1022 with the same values on every run)
    n_new, start = 32, wl.l_past - 32
    out = torch.empty((wl.B, n_new), dtype=torch.int32, device=dev)
    gws = G.generate_workspace(hp, G.BF16, wl.B)

    def gen():
        G.generate_greedy(hp, G.BF16, Wd, ids, wl.B, start, n_new, cache, cap, out, ws=gws, stream=stream)

    gen()
    gen_ms = _timed_loop(gen, max(1, args.decode_steps // 10))
    log(f"[bench] greedy generation {n_new} tokens x {wl.B} sequences from position {start}: "
        f"{gen_ms:.3f} ms, {wl.B * n_new / (gen_ms / 1e3):.4g} tok/s")
    result["generate"] = {"value": round(wl.B * n_new / (gen_ms / 1e3), 1), "unit": "tokens/s",
                          "ms_per_call": round(gen_ms, 4), "n_new": n_new, "from_position": start,
                          "workload": "GPT-2 small greedy generation (gpt2_generate_greedy), B=64, 32 tokens "
                                      "per sequence from position 991 over the decode workload's past"}
    return result


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, ids_np, W, gpu_seqs):
    """The oracle, as it stands, on the host cores: whole sequences of the
    forward workload until about 10 s have passed (the reported value), and
    bounded samples of the other workloads.  Each forward sequence's oracle
    logits are compared with the GPU's logits of the same sequence (parity of
    the timed run)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from gpt_pre_norm_amd.workloads import WORKLOADS, block_inputs, model_inputs, past_for_sequence
    from oracle import gpt2_oracle as O

    affinity = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity)
    cores = max(1, min(affinity, share))
    model = _cpu_model()
    log(f"[bench] cpu oracle baseline on {cores} threads ({affinity} CPUs in the affinity mask; {model})")
    parity = None
    with threadpool_limits(limits=cores):
        n = 0
        errs, g_rows, o_rows = [], [], []
        t0 = time.perf_counter()
        el_fwd = 0.0
        while n < wl.B:
            t1 = time.perf_counter()
            ol, _ = O.model_forward(ids_np[n:n + 1], W, wl.h)
            el_fwd += time.perf_counter() - t1
            if gpu_seqs is not None and n < len(gpu_seqs):
                g = gpu_seqs[n]
                errs.append(float(np.abs(g.astype(np.float64) - ol[0]).max()))
                g_rows.append(g)
                o_rows.append(ol[0])
            n += 1
            if time.perf_counter() - t0 > 10.0:
                break
        if g_rows:
            g, o = np.concatenate(g_rows), np.concatenate(o_rows)
            ga, oa = g.argmax(-1), o.argmax(-1)
            idx = np.arange(len(ga))
            top2 = np.partition(o, -2, axis=-1)[:, -2:]
            wide = (top2[:, 1] - top2[:, 0]) > 6e-2
            parity = {"sequences": len(g_rows), "rows": int(len(ga)), "logits_max_abs_err": max(errs),
                      "tolerance": 3e-2,
                      "argmax_tolerant": float((o[idx, ga] >= o.max(-1) - 3e-2).mean()),
                      "argmax_raw": float((ga == oa).mean()),
                      "argmax_gap_gt_6e-2_rows": int(wide.sum()),
                      "argmax_gap_gt_6e-2_agree": float((ga[wide] == oa[wide]).mean()) if wide.any() else 1.0,
                      "what": "GPU logits of the timed forward vs the oracle, whole sequences"}
            log(f"[bench] parity: {parity}")
        configs = {"gpt2s_fwd_b8_t1024": {"tokens_per_s": round(n * wl.T / el_fwd, 2),
                                          "sample": f"{n} of {wl.B} sequences, full logits", "s": round(el_fwd, 2)}}
        # one fp32 block, d=64, x [2, 8, 64]
        wl1 = WORKLOADS["block_d64_fp32"]
        x1, w1 = block_inputs(wl1)
        reps, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < 1.0:
            O.block_forward(x1, w1, wl1.h)
            reps += 1
        el = time.perf_counter() - t1
        configs["block_d64_fp32"] = {"us_per_call": round(el / reps * 1e6, 1), "sample": f"{reps} calls"}
        # one GPT-2-small block, sequence 0 of 8
        wl2 = WORKLOADS["block_gpt2s_bf16"]
        x2, w2 = block_inputs(wl2)
        t1 = time.perf_counter()
        O.block_forward(x2[:1], w2, wl2.h)
        el = time.perf_counter() - t1
        configs["block_gpt2s_bf16"] = {"tokens_per_s": round(wl2.T / el, 1), "sample": "1 of 8 sequences",
                                       "s": round(el, 2)}
        # the decode step, sequences 0 and 1 of 64 (their past generated outside the timer)
        wl4 = WORKLOADS["gpt2s_decode_b64_p1023"]
        ids4, W4 = model_inputs(wl4)
        el = 0.0
        for b in range(2):
            pb = past_for_sequence(wl4, b)[None]
            t1 = time.perf_counter()
            O.decode_step(ids4[b:b + 1, 0], W4, wl4.h, past=pb)
            el += time.perf_counter() - t1
        configs["gpt2s_decode_b64_p1023"] = {"tokens_per_s": round(2 / el, 2), "sample": "2 of 64 sequences",
                                             "s": round(el, 2)}
    total = time.perf_counter() - t0
    log(f"[bench] cpu oracle configs: {configs} ({total:.1f} s)")
    base = {"value": configs["gpt2s_fwd_b8_t1024"]["tokens_per_s"], "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": model, "affinity_cpus": affinity,
            "sample": f"{n} of {wl.B} sequences of the forward workload (T={wl.T}, full logits), fp64 numpy "
                      f"oracle with {cores} BLAS threads, {el_fwd:.1f} s",
            "configs": configs}
    return base, parity


if __name__ == "__main__":
    main()
