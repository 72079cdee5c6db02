"""Float64 numpy definition of the LLaMA decoder block (test infrastructure only).

Each function follows one passage of the pages; the citation names the page
title and the section or snippet.  Tensor layouts follow the pages' code:
activations [B, S, D], linear weights [out, in] (nn.Linear, y = x W^T),
per-head views [B, S, heads, head_dim], KV cache [max_B, max_S, n_kv_heads,
head_dim].  Nothing here is blocked, fused or reordered beyond the
definitions; functions that take ``rows`` only select which output rows are
evaluated (each output row is defined on its own).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------- widths
def ffn_hidden_dim(dim: int, multiple_of: int, ffn_dim_multiplier: Optional[float]) -> int:
    """FeedForward width rule.

    "LLaMA: Open and Efficient Foundation Language Models" notes, section 3,
    FeedForward.__init__ (called with hidden_dim = 4*dim from TransformerBlock):
    take int(2*hidden/3), scale by the optional multiplier (truncating with
    int), then round up to a multiple of ``multiple_of``.
    """
    hidden = int(2 * (4 * dim) / 3)
    if ffn_dim_multiplier is not None:
        hidden = int(ffn_dim_multiplier * hidden)
    return multiple_of * ((hidden + multiple_of - 1) // multiple_of)


# --------------------------------------------------------------------------- RMSNorm
def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * weight.

    Same notes, section 3, class RMSNorm (_norm and forward); eps sits inside
    the square root as in the code (the formula printed in "灵哥讲llama3(中)",
    RMSNorm section, puts it outside; the code's form is taken).  No mean is
    subtracted and there is no bias.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


# --------------------------------------------------------------------------- RoPE
def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """theta_i = theta^(-2i/d) for i = 0 .. d/2-1.

    Same notes, section 3, precompute_freqs_cis: arange(0, dim, 2)[:dim//2]/dim
    as the exponent of 1/theta.
    """
    i = np.arange(head_dim // 2, dtype=np.float64)
    return 1.0 / (float(theta) ** (2.0 * i / head_dim))


def rope_angles(head_dim: int, positions: Sequence[int], theta: float) -> np.ndarray:
    """Angle table: outer(position, theta_i), shape [len(positions), d/2] (precompute_freqs_cis)."""
    return np.outer(np.asarray(positions, dtype=np.float64), rope_inv_freq(head_dim, theta))


def freqs_cis(head_dim: int, end: int, theta: float) -> np.ndarray:
    """complex table e^{i * p * theta_i}, [end, d/2] (precompute_freqs_cis with torch.polar)."""
    ang = rope_angles(head_dim, range(end), theta)
    return np.cos(ang) + 1j * np.sin(ang)


def apply_rope(u: np.ndarray, positions: Sequence[int], theta: float) -> np.ndarray:
    """Rotate each interleaved pair (u[2i], u[2i+1]) by the angle p*theta_i.

    Same notes, section 3, apply_rotary_emb: the last axis is viewed as complex
    numbers (real = even element, imag = odd element) and multiplied by
    e^{i p theta_i}; written out, (a, b) -> (a cos - b sin, a sin + b cos),
    the 2x2 rotation of the linkmax.top walkthrough, section 2.3.
    ``u`` is [B, S, heads, d]; ``positions`` has length S.
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    ang = rope_angles(d, positions, theta)           # [S, d/2]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    a = u[..., 0::2]
    b = u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# --------------------------------------------------------------------------- attention
def repeat_kv(x: np.ndarray, n_rep: int) -> np.ndarray:
    """[B, T, Hkv, d] -> [B, T, Hkv*n_rep, d]; head h reads kv head h // n_rep (repeat_kv)."""
    if n_rep == 1:
        return x
    B, T, Hkv, d = x.shape
    return np.broadcast_to(x[:, :, :, None, :], (B, T, Hkv, n_rep, d)).reshape(B, T, Hkv * n_rep, d)


def causal_mask(seqlen: int, start_pos: int) -> np.ndarray:
    """Additive mask [S, start_pos + S]: -inf where key t > start_pos + s, else 0.

    "灵哥讲llama3(中)", Transformer forward: triu(-inf, diagonal=1) on the
    new block, stacked to the right of start_pos zero columns.  No mask when
    seqlen == 1 (the same code builds one only when seqlen > 1).
    """
    T = start_pos + seqlen
    s = np.arange(seqlen)[:, None]
    t = np.arange(T)[None, :]
    return np.where(t > start_pos + s, -np.inf, 0.0)


def softmax(z: np.ndarray) -> np.ndarray:
    """Row softmax over the last axis (subtracting the row max leaves the value unchanged)."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_probs(xq: np.ndarray, keys: np.ndarray, start_pos: int,
                    rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """softmax(q k^T / sqrt(d) + mask) per head: [B, H, len(rows), T].

    Same notes, section 3, Attention.forward: scores = xq @ keys^T / sqrt(head_dim),
    plus the causal mask, softmax over keys.  ``keys`` is the cache slice
    [:B, :start_pos+S] already expanded to all H heads.
    """
    B, S, H, d = xq.shape
    rows = np.arange(S) if rows is None else np.asarray(rows)
    q = np.transpose(xq[:, rows], (0, 2, 1, 3))                   # [B, H, R, d]
    k = np.transpose(keys, (0, 2, 1, 3))                          # [B, H, T, d]
    scores = np.matmul(q, np.transpose(k, (0, 1, 3, 2))) / math.sqrt(d)
    if S > 1:
        scores = scores + causal_mask(S, start_pos)[rows][None, None]
    return softmax(scores)


def gqa_attention(xq: np.ndarray, cache_k: np.ndarray, cache_v: np.ndarray, start_pos: int,
                  rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Grouped-query attention over the cache: output [B, len(rows), H*d].

    Same notes, section 3, Attention.forward after the cache write: keys and
    values are cache[:B, :start_pos+S], expanded with repeat_kv (so q head h
    uses kv head h // n_rep), softmax(q k^T/sqrt(d) + mask) @ v, heads
    concatenated.
    """
    B, S, H, d = xq.shape
    T = start_pos + S
    Hkv = cache_k.shape[2]
    n_rep = H // Hkv
    keys = repeat_kv(np.asarray(cache_k[:B, :T], dtype=np.float64), n_rep)
    values = repeat_kv(np.asarray(cache_v[:B, :T], dtype=np.float64), n_rep)
    p = attention_probs(np.asarray(xq, dtype=np.float64), keys, start_pos, rows)   # [B, H, R, T]
    v = np.transpose(values, (0, 2, 1, 3))                        # [B, H, T, d]
    o = np.matmul(p, v)                                           # [B, H, R, d]
    R = o.shape[2]
    return np.transpose(o, (0, 2, 1, 3)).reshape(B, R, H * d)


# --------------------------------------------------------------------------- FFN
def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a) = a / (1 + e^-a) (SwiGLU section of "LLaMa-1/2/3 原理+源码")."""
    return a / (1.0 + np.exp(-a))


def swiglu_ffn(x: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """w2(silu(w1 x) * w3 x) with nn.Linear weights (same notes, section 3, FeedForward.forward)."""
    x = np.asarray(x, dtype=np.float64)
    a = x @ np.asarray(w1, dtype=np.float64).T
    b = x @ np.asarray(w3, dtype=np.float64).T
    return (silu(a) * b) @ np.asarray(w2, dtype=np.float64).T


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """nn.Linear without bias: y = x W^T, W stored [out, in]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


# --------------------------------------------------------------------------- block
def block_forward(x: np.ndarray, w: Dict[str, np.ndarray], cache_k: np.ndarray, cache_v: np.ndarray,
                  start_pos: int, n_heads: int, n_kv_heads: int, norm_eps: float, rope_theta: float,
                  rows: Optional[Sequence[int]] = None, trace: Optional[dict] = None) -> np.ndarray:
    """One pre-norm decoder block; mutates cache_k/cache_v at [:B, start_pos:start_pos+S].

    Same notes, section 3, TransformerBlock.forward:
        h   = x + Attention(RMSNorm(x))          (attention_norm, wq/wk/wv, RoPE on q and k,
                                                  cache write, GQA attention, wo)
        out = h + FeedForward(RMSNorm(h))        (ffn_norm, w2(silu(w1 .) * w3 .))
    The cache receives k after RoPE and v as projected.  ``rows`` selects which
    output rows (sequence positions within this call) are evaluated; k and v
    are always computed for all S new positions, since the cache needs them.
    ``trace``, when given, receives the intermediate tensors by name.
    """
    x = np.asarray(x, dtype=np.float64)
    B, S, D = x.shape
    pos = list(range(start_pos, start_pos + S))
    rows_a = np.arange(S) if rows is None else np.asarray(rows)
    xn = rms_norm(x, w["attention_norm"], norm_eps)
    d = D // n_heads
    k = linear(xn, w["wk"]).reshape(B, S, n_kv_heads, d)
    v = linear(xn, w["wv"]).reshape(B, S, n_kv_heads, d)
    k = apply_rope(k, pos, rope_theta)
    cache_k[:B, start_pos:start_pos + S] = k
    cache_v[:B, start_pos:start_pos + S] = v
    q = linear(xn[:, rows_a], w["wq"]).reshape(B, len(rows_a), n_heads, d)
    q = apply_rope(q, [pos[r] for r in rows_a], rope_theta)
    # attention needs q at the selected rows only; place them in an [B, S, H, d]
    # array so the mask rows line up with their sequence positions.
    q_full = np.zeros((B, S, n_heads, d))
    q_full[:, rows_a] = q
    o = gqa_attention(q_full, cache_k, cache_v, start_pos, rows_a)          # [B, R, H*d]
    h = x[:, rows_a] + linear(o, w["wo"])
    hn = rms_norm(h, w["ffn_norm"], norm_eps)
    out = h + swiglu_ffn(hn, w["w1"], w["w3"], w["w2"])
    if trace is not None:
        trace.update(xn=xn[:, rows_a], q=q, k=k, v=v, o=o, h=h, hn=hn, out=out)
    return out


def stack_forward(tok: np.ndarray, embed: np.ndarray, layers: Sequence[Dict[str, np.ndarray]],
                  norm_w: np.ndarray, w_out: np.ndarray, caches: Sequence, start_pos: int,
                  n_heads: int, n_kv_heads: int, norm_eps: float, rope_theta: float):
    """Whole-model forward for one call; logits of the last position only and the greedy token.

    linkmax.top walkthrough, section 3.2.2 (Transformer.forward: embedding,
    layers, norm, output on h[:, -1]) and section 3.3 (generate: argmax when
    temperature is 0; the lowest index wins exact ties, as numpy's argmax).
    Returns (logits [B, vocab], next_token [B]).
    """
    h = np.asarray(embed, dtype=np.float64)[np.asarray(tok)]
    for lw, (ck, cv) in zip(layers, caches):
        h = block_forward(h, lw, ck, cv, start_pos, n_heads, n_kv_heads, norm_eps, rope_theta)
    hl = rms_norm(h[:, -1], norm_w, norm_eps)
    logits = linear(hl, w_out)
    return logits, np.argmax(logits, axis=-1)
