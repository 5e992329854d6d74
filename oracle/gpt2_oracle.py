"""CPU oracle for the GPT-2 pre-norm decoder forward and its cached decode step.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
definition that the HIP path is checked against.  Only the tests, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
it; the library in ``gpt_pre_norm_amd`` never calls it and shares no code with it.

Everything is computed in float64 with numpy.  Inputs are whatever arrays the
caller passes (the bf16 workloads pass their bf16-rounded values), upcast to
float64 on entry.  The only library primitive used for a step is the matrix
product; every other step is written out as the pages define it.

Sources (web pages, cited by title and section):
* "Decoder Block" (GPT-2, AI Engineer Exhaustive), sections "Overview" and
  "How it works": pre-norm block with two residual adds, LN1/LN2 with eps 1e-5,
  causal multi-head attention with a fused QKV projection, 4d GELU MLP, final ln_f.
* "Decoder-only" (CodeBlanks), "The decoder-only architecture", "GPT-2 small:
  124 million" and its "Expected output": tied head and the parameter-count formula.
* "GPT-2 Block - TorchCode", "Reference Solution": per-head scaling by
  1/sqrt(d_k), the upper-triangle mask, softmax, head merge.
* "GPT-2 Transformer block" (Open Model Atlas), excerpt of ``norm()``: mean,
  biased variance of deviations, rsqrt(s + eps), then gain and bias.
* "Full Forward Pass" (GPT-2, AI Engineer Exhaustive), "How it works": the
  embedding sum with positions offset by the cache length, the stacked
  ``present`` of shape [B, L, 2, h, T, d_h], ln_f and the tied projection.

Readings where the pages are silent:
* GELU is the tanh approximation (the pages only name ``gelu``).
* Key m is visible to query i iff m <= l_past + i (absolute positions).
* Weights of every linear layer are stored [out, in]; y = x W^T + b.
* The fused QKV output is split q | k | v along the last axis; head j takes the
  contiguous columns [j*d_h, (j+1)*d_h) of each.
* Positions must satisfy l_past + T <= n_ctx ("strictly below n_ctx").
"""
from __future__ import annotations

import numpy as np

EPS = 1e-5
BLOCK_KEYS = ("ln1_g", "ln1_b", "attn_w", "attn_b", "proj_w", "proj_b",
              "ln2_g", "ln2_b", "fc_w", "fc_b", "fc2_w", "fc2_b")


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------------ parameters

def block_param_shapes(d: int) -> dict:
    """Shapes of one block's parameters ("Decoder Block", How it works; the
    per-layer terms of the count in "Decoder-only", GPT-2 small)."""
    return {
        "ln1_g": (d,), "ln1_b": (d,),
        "attn_w": (3 * d, d), "attn_b": (3 * d,),
        "proj_w": (d, d), "proj_b": (d,),
        "ln2_g": (d,), "ln2_b": (d,),
        "fc_w": (4 * d, d), "fc_b": (4 * d,),
        "fc2_w": (d, 4 * d), "fc2_b": (d,),
    }


def model_param_shapes(n_vocab: int, n_ctx: int, d: int, n_layer: int) -> dict:
    """Shapes of the whole model's parameters, tied head (no separate output
    matrix) and ln_f included ("Full Forward Pass", How it works)."""
    shapes = {"wte": (n_vocab, d), "wpe": (n_ctx, d), "lnf_g": (d,), "lnf_b": (d,)}
    for layer in range(n_layer):
        for k, s in block_param_shapes(d).items():
            shapes[f"h{layer}.{k}"] = s
    return shapes


def count(shapes: dict) -> int:
    return int(sum(int(np.prod(s)) for s in shapes.values()))


# ------------------------------------------------------------------ the steps

def layer_norm(x, g, b, eps: float = EPS):
    """LayerNorm over the last axis (Open Model Atlas excerpt of norm(); "Decoder
    Block", How it works): u = mean(x), s = mean((x - u)^2), then
    (x - u) / sqrt(s + eps), then times the gain and plus the bias."""
    x = _f64(x)
    u = x.mean(axis=-1, keepdims=True)
    s = ((x - u) ** 2).mean(axis=-1, keepdims=True)
    return (x - u) / np.sqrt(s + eps) * _f64(g) + _f64(b)


def gelu(x):
    """GELU, tanh approximation (Hendrycks & Gimpel 2016):
    0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = _f64(x)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def linear(x, w, b=None):
    """y = x W^T (+ b), W stored [out, in]."""
    y = _f64(x) @ _f64(w).T
    return y if b is None else y + _f64(b)


def split_heads(t, n_head: int):
    """[B, T, d] -> [B, h, T, d_h]; head j holds columns j*d_h .. (j+1)*d_h - 1."""
    B, T, d = t.shape
    return t.reshape(B, T, n_head, d // n_head).transpose(0, 2, 1, 3)


def merge_heads(t):
    """[B, h, T, d_h] -> [B, T, h*d_h], the inverse of split_heads."""
    B, h, T, dh = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, T, h * dh)


def causal_attention(q, k, v, l_past: int = 0):
    """Scaled dot-product attention with the causal mask ("GPT-2 Block -
    TorchCode", Reference Solution; "Decoder Block", How it works).

    q: [B, h, T, d_h]; k, v: [B, h, l_past + T, d_h] (cached keys first).
    Query i sits at absolute position l_past + i and sees keys m <= l_past + i.
    Each row: scores / sqrt(d_h), subtract the row max, exponentiate, normalise,
    weight the values.  Masked keys get weight exactly 0.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, dh = q.shape[2], q.shape[3]
    Tk = k.shape[2]
    assert Tk == l_past + T
    scores = (q @ k.transpose(0, 1, 3, 2)) / np.sqrt(dh)
    qpos = l_past + np.arange(T)[:, None]
    kpos = np.arange(Tk)[None, :]
    visible = kpos <= qpos
    scores = np.where(visible, scores, -np.inf)
    scores = scores - scores.max(axis=-1, keepdims=True)
    p = np.exp(scores)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v


def attention(a, w: dict, n_head: int, past=None):
    """Attn sub-block: fused c_attn, head split, optional past concat, causal
    attention, head merge, c_proj ("Full Forward Pass", How it works).

    a: LN1 output [B, T, d].  past: [B, 2, h, T_past, d_h] or None.
    Returns (output [B, T, d], present [B, 2, h, T, d_h])."""
    d = a.shape[-1]
    qkv = linear(a, w["attn_w"], w["attn_b"])
    q = split_heads(qkv[..., 0:d], n_head)
    k = split_heads(qkv[..., d:2 * d], n_head)
    v = split_heads(qkv[..., 2 * d:3 * d], n_head)
    present = np.stack([k, v], axis=1)
    l_past = 0
    if past is not None:
        past = _f64(past)
        l_past = past.shape[3]
        k = np.concatenate([past[:, 0], k], axis=2)
        v = np.concatenate([past[:, 1], v], axis=2)
    o = merge_heads(causal_attention(q, k, v, l_past))
    return linear(o, w["proj_w"], w["proj_b"]), present


def mlp(a, w: dict):
    """MLP sub-block: c_fc to 4d, GELU, c_proj back to d."""
    return linear(gelu(linear(a, w["fc_w"], w["fc_b"])), w["fc2_w"], w["fc2_b"])


def block_forward(x, w: dict, n_head: int, past=None, eps: float = EPS):
    """One pre-norm block ("Decoder Block", How it works; Open Model Atlas block
    excerpts): x <- x + Attn(LN1 x); x <- x + MLP(LN2 x).  Both adds go onto the
    un-normalised stream.  Returns (y, present)."""
    x = _f64(x)
    a, present = attention(layer_norm(x, w["ln1_g"], w["ln1_b"], eps), w, n_head, past)
    x = x + a
    x = x + mlp(layer_norm(x, w["ln2_g"], w["ln2_b"], eps), w)
    return x, present


def embed(ids, wte, wpe, l_past: int = 0):
    """H0 = wte[ids] + wpe[l_past + t] ("Full Forward Pass", How it works)."""
    ids = np.asarray(ids)
    T = ids.shape[1]
    n_ctx = wpe.shape[0]
    if l_past + T > n_ctx:
        raise ValueError("positions must stay below n_ctx")
    if ids.min() < 0 or ids.max() >= wte.shape[0]:
        raise ValueError("token id out of range")
    pos = l_past + np.arange(T)
    return _f64(wte)[ids] + _f64(wpe)[pos][None, :, :]


def model_forward(ids, W: dict, n_head: int, past=None, logit_rows=None, eps: float = EPS):
    """Full forward ("Full Forward Pass", How it works): embed, L blocks, ln_f,
    tied head logits = LN_f(H) wte^T.

    ids: [B, T] int.  past: [B, L, 2, h, T_past, d_h] or None.
    logit_rows: optional 1-D array of flat row indices b*T + t; when given only
    those rows of the head are computed (the head is row-wise) and logits is
    [len(logit_rows), V].  Returns (logits [B, T, V], present [B, L, 2, h, T, d_h])."""
    ids = np.asarray(ids)
    B, T = ids.shape
    l_past = 0 if past is None else past.shape[4]
    h = embed(ids, W["wte"], W["wpe"], l_past)
    presents = []
    for layer, w in enumerate(W["blocks"]):
        p = None if past is None else past[:, layer]
        h, pres = block_forward(h, w, n_head, p, eps)
        presents.append(pres)
    present = np.stack(presents, axis=1)
    z = layer_norm(h, W["lnf_g"], W["lnf_b"], eps)
    d = z.shape[-1]
    if logit_rows is not None:
        logits = z.reshape(B * T, d)[np.asarray(logit_rows)] @ _f64(W["wte"]).T
    else:
        logits = (z.reshape(B * T, d) @ _f64(W["wte"]).T).reshape(B, T, -1)
    return logits, present


def decode_step(ids, W: dict, n_head: int, past, eps: float = EPS):
    """Cached decode ("Full Forward Pass", How it works, last paragraph): feed
    only the newest token (ids [B]) plus the stacked present of the earlier
    steps; returns (logits [B, 1, V], present of the new token
    [B, L, 2, h, 1, d_h])."""
    ids = np.asarray(ids).reshape(-1, 1)
    return model_forward(ids, W, n_head, past=past, eps=eps)


def next_token_loss(logits, targets):
    """Next-token cross-entropy that callers take of the logits ("Full Forward
    Pass", How it works): per position, log(sum_n exp(logit_n)) -
    logit_target, the log-sum-exp taken about the row maximum.
    logits [..., V]; targets [...] ints in [0, V).  Returns [...] float64."""
    z = _f64(logits)
    t = np.asarray(targets)
    mx = z.max(axis=-1, keepdims=True)
    lse = mx[..., 0] + np.log(np.exp(z - mx).sum(axis=-1))
    return lse - np.take_along_axis(z, t[..., None], axis=-1)[..., 0]
