"""Algorithmic work per kernel launch and the MI355X peaks it is priced against.

Flops count what the method must compute (2 per multiply-add; causal
attention counts only the T(T+1)/2 visible query-key pairs).  Bytes count what
the step must move to or from HBM at least once (operands read, results
written), independent of how a kernel tiles or re-reads them.
"""
from __future__ import annotations

PEAK_BF16_FLOPS = 2.5e15   # dense bf16 MFMA, MI355X published figure
PEAK_HBM_BYTES = 8.0e12    # HBM3E, MI355X published figure
RIDGE = PEAK_BF16_FLOPS / PEAK_HBM_BYTES


def kernel_work(kind: str, *, B: int, T: int, d: int, h: int, V: int, l_past: int = 0,
                act: int = 2) -> tuple[float, float]:
    """(flops, bytes) of one launch of a kernel kind in the bf16 path."""
    M = B * T
    dh = d // h

    def gemm(N, K, out_bytes, extra_read=0):
        flops = 2.0 * M * N * K
        byt = (M * K + N * K) * act + M * N * out_bytes + N * act + extra_read
        return flops, byt

    if kind == "embed":
        return 0.0, M * 4 + 2 * M * d * act + M * d * 4
    if kind == "layernorm":
        return 8.0 * M * d, M * d * 4 + M * d * act + 2 * d * act
    if kind == "gemm_c_attn":
        return gemm(3 * d, d, act)
    if kind == "gemm_attn_c_proj":
        return gemm(d, d, 4, extra_read=M * d * 4)
    if kind == "gemm_c_fc":
        return gemm(4 * d, d, act)
    if kind == "gemm_mlp_c_proj":
        return gemm(d, 4 * d, 4, extra_read=M * d * 4)
    if kind == "gemm_lm_head":
        return gemm(V, d, 4)
    if kind == "attn_prefill":
        pairs = B * h * (T * (T + 1) // 2 + l_past * T)
        flops = 4.0 * pairs * dh
        byt = 4.0 * M * d * act  # q, k, v read once, o written once
        return flops, byt
    if kind == "attn_decode":
        nk = l_past + 1
        flops = 4.0 * B * h * nk * dh
        byt = 2.0 * B * h * nk * dh * act + 2 * B * d * act  # K and V rows, q in, o out
        return flops, byt
    raise KeyError(kind)


def bound_of(flops: float, byt: float) -> str:
    return "mfma" if byt == 0 or flops / byt >= RIDGE else "hbm"


def model_flops(B: int, T: int, d: int, h: int, L: int, V: int) -> float:
    """Algorithmic flops of one uncached forward (causal attention, tied head)."""
    M = B * T
    gemms = 2.0 * M * d * (3 * d + d + 4 * d + 4 * d)
    attn = 2.0 * d * T * (T + 1) * B
    return L * (gemms + attn) + 2.0 * M * V * d


def decode_bytes(B: int, d: int, h: int, L: int, V: int, l_past: int, act: int = 2) -> float:
    """Algorithmic HBM bytes of one cached decode step: the cache read for
    positions 0..l_past, every weight read once, the new K/V and the logits written."""
    kv = 2.0 * B * L * (l_past + 1) * d * act
    per_layer_w = (3 * d * d + d * d + 4 * d * d + 4 * d * d) * act + (3 * d + d + 4 * d + d + 4 * d) * act
    weights = L * per_layer_w + V * d * act + 2 * d * act
    logits = B * V * 4.0
    gathered = B * d * act * 2  # wte and wpe rows of the new tokens
    return kv + weights + logits + gathered
