"""The synthetic workloads: sizes, seeds and the input recipe of each.

Names describe the workload; the inputs come from ``synth`` (seeded,
counter-based) and are identical for the HIP path and the oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import synth

FP32, BF16 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "block" | "forward" | "decode"
    mode: int            # FP32 | BF16
    n_vocab: int
    n_ctx: int
    d: int
    h: int
    L: int
    B: int
    T: int               # new tokens per sequence (1 for decode)
    l_past: int = 0      # decode: cached positions
    seed: int = 0
    resid_scale: float = 1.0
    affine: str = "default"
    note: str = ""

    @property
    def dh(self) -> int:
        return self.d // self.h

    @property
    def tokens(self) -> int:
        return self.B * self.T


# Block: GPT-2 small width with residual projections scaled by 1/sqrt(2*12).
WORKLOADS = {
    "block_d64_fp32": Workload(
        "block_d64_fp32", "block", FP32, 0, 1024, 64, 4, 1, 2, 8, seed=0,
        note="one block, fp32, d=64, 4 heads, x [2, 8, 64] ~ N(0,1), weights N(0, 0.02)"),
    "block_gpt2s_bf16": Workload(
        "block_gpt2s_bf16", "block", BF16, 0, 1024, 768, 12, 1, 8, 1024, seed=1,
        resid_scale=1 / math.sqrt(24),
        note="one GPT-2-small block, bf16, x [8, 1024, 768] ~ N(0,1)"),
    "gpt2s_fwd_b8_t1024": Workload(
        "gpt2s_fwd_b8_t1024", "forward", BF16, 50257, 1024, 768, 12, 12, 8, 1024, seed=2,
        resid_scale=1 / math.sqrt(24),
        note="GPT-2 small uncached forward, bf16, ids [8, 1024] uniform, logits fp32 [8, 1024, 50257]"),
    "gpt2s_decode_b64_p1023": Workload(
        "gpt2s_decode_b64_p1023", "decode", BF16, 50257, 1024, 768, 12, 12, 64, 1, l_past=1023, seed=3,
        resid_scale=1 / math.sqrt(24),
        note="GPT-2 small cached decode, bf16, 64 sequences at position 1023, past ~ N(0,1)"),
    # The other depths of the published table, L = 24 and 36; the pages print
    # no widths for them: d = 1024 (16 heads) and d = 1280 (20 heads), head
    # width 64 and a 4d MLP as at every depth, residual projections scaled by
    # 1/sqrt(2L), B = 4 like the 48-layer workload.
    "gpt2_l24_d1024_fwd_b4_t1024": Workload(
        "gpt2_l24_d1024_fwd_b4_t1024", "forward", BF16, 50257, 1024, 1024, 16, 24, 4, 1024, seed=5,
        resid_scale=1 / math.sqrt(48),
        note="24 layers, d=1024, 16 heads, bf16, ids [4, 1024], logits fp32 [4, 1024, 50257]"),
    "gpt2_l36_d1280_fwd_b4_t1024": Workload(
        "gpt2_l36_d1280_fwd_b4_t1024", "forward", BF16, 50257, 1024, 1280, 20, 36, 4, 1024, seed=6,
        resid_scale=1 / math.sqrt(72),
        note="36 layers, d=1280, 20 heads, bf16, ids [4, 1024], logits fp32 [4, 1024, 50257]"),
    "gpt2_l48_d1600_fwd_b4_t1024": Workload(
        "gpt2_l48_d1600_fwd_b4_t1024", "forward", BF16, 50257, 1024, 1600, 25, 48, 4, 1024, seed=4,
        resid_scale=1 / math.sqrt(96),
        note="48 layers, d=1600, 25 heads, bf16, ids [4, 1024], logits fp32 [4, 1024, 50257]"),
}


def block_inputs(wl: Workload, affine: str | None = None):
    bf = wl.mode == BF16
    x = synth.hidden_input((wl.B, wl.T, wl.d), wl.seed, bf16=bf)
    w = synth.block_weights(wl.d, wl.seed, 0, resid_scale=wl.resid_scale,
                            affine=affine or wl.affine, bf16=bf)
    return x, w


def model_inputs(wl: Workload, affine: str | None = None):
    bf = wl.mode == BF16
    W = synth.model_weights(wl.n_vocab, wl.n_ctx, wl.d, wl.L, wl.seed, affine=affine or wl.affine,
                            bf16=bf, resid_scale=wl.resid_scale)
    ids = synth.ids_input((wl.B, wl.T), wl.n_vocab, wl.seed)
    return ids, W


def past_shape(wl: Workload):
    """The filled part of the cache, [B, L, 2, h, l_past, d_h]."""
    return (wl.B, wl.L, 2, wl.h, wl.l_past, wl.dh)


def past_for_sequence(wl: Workload, b: int) -> np.ndarray:
    """Sequence b's slice of the past ([L, 2, h, l_past, d_h], fp32 values of the mode)."""
    per_seq = wl.L * 2 * wl.h * wl.l_past * wl.dh
    flat = synth.past_normal((per_seq,), wl.seed, start=b * per_seq, bf16=wl.mode == BF16)
    return flat.reshape(wl.L, 2, wl.h, wl.l_past, wl.dh)
