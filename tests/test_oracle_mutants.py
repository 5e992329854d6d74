"""Plants plausible mistakes in the CPU oracle and checks that the pins catch each.

A mutant replaces one oracle function for the duration of a test (CPU only).
If every pin still passes under a mutant, the pins cannot tell that mistake
from the correct oracle, and this test fails.
"""
import numpy as np
import pytest
from scipy.special import erf

from oracle import gpt2_oracle as O
from oracle_pins import PINS

_orig = {k: getattr(O, k) for k in ("layer_norm", "gelu", "causal_attention", "attention",
                                    "block_forward", "embed", "model_forward", "split_heads",
                                    "merge_heads", "linear", "block_param_shapes")}


def m_gelu_erf(x):
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1 + erf(x / np.sqrt(2)))


def m_ln_unbiased(x, g, b, eps=1e-5):
    x = np.asarray(x, np.float64)
    u = x.mean(-1, keepdims=True)
    s = ((x - u) ** 2).sum(-1, keepdims=True) / (x.shape[-1] - 1)
    return (x - u) / np.sqrt(s + eps) * g + b


def m_ln_eps_outside(x, g, b, eps=1e-5):
    x = np.asarray(x, np.float64)
    u = x.mean(-1, keepdims=True)
    s = ((x - u) ** 2).mean(-1, keepdims=True)
    return (x - u) / (np.sqrt(s) + eps) * g + b


def m_ln_affine_swapped(x, g, b, eps=1e-5):
    return _orig["layer_norm"](x, b, g, eps)


def _attn_variant(scale=None, strict=False, nomask=False):
    def f(q, k, v, l_past=0):
        q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
        T, dh = q.shape[2], q.shape[3]
        Tk = k.shape[2]
        sc = q @ k.transpose(0, 1, 3, 2) * (1 / np.sqrt(dh) if scale is None else scale(dh))
        qpos = l_past + np.arange(T)[:, None]
        kpos = np.arange(Tk)[None, :]
        vis = np.ones((T, Tk), bool) if nomask else ((kpos < qpos) if strict else (kpos <= qpos))
        sc = np.where(vis, sc, -np.inf)
        sc = sc - sc.max(-1, keepdims=True)
        p = np.exp(sc)
        return (p / p.sum(-1, keepdims=True)) @ v
    return f


def m_attn_qkv_order(a, w, n_head, past=None):
    # splits the fused projection as q | v | k
    d = a.shape[-1]
    w2 = dict(w)
    W, bb = np.asarray(w["attn_w"]), np.asarray(w["attn_b"])
    w2["attn_w"] = np.concatenate([W[:d], W[2 * d:], W[d:2 * d]])
    w2["attn_b"] = np.concatenate([bb[:d], bb[2 * d:], bb[d:2 * d]])
    return _orig["attention"](a, w2, n_head, past)


def m_split_interleaved(t, n_head):
    B, T, d = t.shape
    return t.reshape(B, T, d // n_head, n_head).transpose(0, 3, 1, 2)


def m_merge_interleaved(t):
    B, h, T, dh = t.shape
    return t.transpose(0, 2, 3, 1).reshape(B, T, h * dh)


def m_block_post_norm(x, w, n_head, past=None, eps=1e-5):
    x = np.asarray(x, np.float64)
    a, present = O.attention(x, w, n_head, past)
    x = O.layer_norm(x + a, w["ln1_g"], w["ln1_b"], eps)
    x = O.layer_norm(x + O.mlp(x, w), w["ln2_g"], w["ln2_b"], eps)
    return x, present


def m_block_shared_ln(x, w, n_head, past=None, eps=1e-5):
    w2 = dict(w)
    w2["ln2_g"], w2["ln2_b"] = w["ln1_g"], w["ln1_b"]
    return _orig["block_forward"](x, w2, n_head, past, eps)


def m_block_no_attn_residual(x, w, n_head, past=None, eps=1e-5):
    x = np.asarray(x, np.float64)
    a, present = O.attention(O.layer_norm(x, w["ln1_g"], w["ln1_b"], eps), w, n_head, past)
    x = a
    return x + O.mlp(O.layer_norm(x, w["ln2_g"], w["ln2_b"], eps), w), present


def m_linear_no_bias(x, w, b=None):
    return _orig["linear"](x, w, None)


def m_embed_no_offset(ids, wte, wpe, l_past=0):
    return _orig["embed"](ids, wte, wpe, 0)


def m_model_no_lnf(ids, W, n_head, past=None, logit_rows=None, eps=1e-5):
    # the last LayerNorm call (ln_f) returns its input unchanged
    saved = O.layer_norm
    calls = {"n": 0}
    n_ln = 2 * len(W["blocks"]) + 1

    def ln(x, g, b, eps=1e-5):
        calls["n"] += 1
        if calls["n"] == n_ln:
            return np.asarray(x, np.float64)
        return saved(x, g, b, eps)
    O.layer_norm = ln
    try:
        return _orig["model_forward"](ids, W, n_head, past, logit_rows, eps)
    finally:
        O.layer_norm = saved


def m_block_shapes_untied(d):
    s = dict(_orig["block_param_shapes"](d))
    s["fc_b"] = (d,)
    return s


MUTANTS = {
    "gelu_erf": ("gelu", m_gelu_erf),
    "ln_unbiased_var": ("layer_norm", m_ln_unbiased),
    "ln_eps_outside_sqrt": ("layer_norm", m_ln_eps_outside),
    "ln_gain_bias_swapped": ("layer_norm", m_ln_affine_swapped),
    "attn_no_scale": ("causal_attention", _attn_variant(scale=lambda dh: 1.0)),
    "attn_scale_1_over_dh": ("causal_attention", _attn_variant(scale=lambda dh: 1.0 / dh)),
    "attn_mask_strict": ("causal_attention", _attn_variant(strict=True)),
    "attn_no_mask": ("causal_attention", _attn_variant(nomask=True)),
    "qkv_split_order": ("attention", m_attn_qkv_order),
    "head_split_interleaved": ("split_heads", m_split_interleaved),
    "head_merge_interleaved": ("merge_heads", m_merge_interleaved),
    "post_norm": ("block_forward", m_block_post_norm),
    "shared_ln_params": ("block_forward", m_block_shared_ln),
    "no_attn_residual": ("block_forward", m_block_no_attn_residual),
    "dropped_biases": ("linear", m_linear_no_bias),
    "positions_not_offset": ("embed", m_embed_no_offset),
    "no_final_ln": ("model_forward", m_model_no_lnf),
    "wrong_param_layout": ("block_param_shapes", m_block_shapes_untied),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError, TypeError) as e:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
