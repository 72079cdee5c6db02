"""Seeded synthetic inputs for the LLaMA decoder-block forward pass.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds no part of the block's arithmetic: it only names the
workloads (shapes and hyper-parameters) and draws seeded random tensors for
them.  The shapes follow the ModelArgs fields of the consolidated single-GPU
code ("LLaMA: Open and Efficient Foundation Language Models" notes, section
3 "代码实现", ModelArgs) and the model-size table of "LLaMA v1/2模型结构总览".

Recipe (the same for every workload):
  * one ``torch.Generator`` (CPU, mt19937) per tensor, seeded from
    ``SeedSequence(1234, spawn_key=(workload_id, layer, tensor_id))``;
  * ``torch.randn`` in float32, times the stated standard deviation
    (0.02 for linear weights, embedding and LM head; 1 for activations and
    pre-filled cache rows);
  * for bf16 workloads the float32 draw is rounded to bfloat16 with
    round-to-nearest-even (``tensor.to(torch.bfloat16)``);
  * RMSNorm weights are ones (the pages initialise them to ones, and the five
    workloads state unit weights).  A test workload may instead draw them,
    seeded per norm and per layer, so that a swapped or dropped gain changes
    the result: ``norm_gains="normal"`` gives 1 + N(0, 0.2^2);
    ``norm_gains="pow2"`` gives 2^k with k uniform in {-1, 0, 1}, for which
    x * g is exact in bf16 (the 32-layer tests use it: there the bf16 rounding
    of x * g, which the per-block tests cover with "normal" gains, would take
    most of the error budget of a layer fed with the small embedding rows);
  * token ids are uniform in [0, vocab).

Tensor ids: 0 x_prefill, 1 x_decode, 2..8 wq wk wv wo w1 w2 w3,
9/10 pre-filled cache k/v, 11 embedding, 12 output projection, 13 token ids,
14/15 attention_norm / ffn_norm gains, 16 final-norm gain, 20 scratch for tests.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np
import torch

BASE_SEED = 1234

T_X_PREFILL, T_X_DECODE = 0, 1
T_WQ, T_WK, T_WV, T_WO, T_W1, T_W2, T_W3 = 2, 3, 4, 5, 6, 7, 8
T_CACHE_K, T_CACHE_V = 9, 10
T_EMBED, T_OUTPUT, T_TOKENS = 11, 12, 13
T_ATTN_NORM, T_FFN_NORM, T_FINAL_NORM = 14, 15, 16
T_TEST = 20

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: model hyper-parameters plus the run's shape."""
    wid: int
    name: str
    dtype: str                 # "f32" or "bf16"
    dim: int
    n_heads: int
    n_kv_heads: int
    ffn_hidden: int            # the width the workload states
    multiple_of: int
    ffn_dim_multiplier: Optional[float]
    norm_eps: float
    rope_theta: float
    batch: int
    prefill_len: int           # tokens in the prefill call (0: none)
    decode_steps: int          # one-token calls after the prefill
    cache_prefill: int = 0     # positions pre-filled with N(0,1) (decode-only workload)
    n_layers: int = 1
    vocab_size: int = 0
    norm_gains: str = "ones"    # RMSNorm weights: "ones", "normal" or "pow2" (see the module docstring)

    @property
    def head_dim(self) -> int:
        return self.dim // self.n_heads

    @property
    def max_seq_len(self) -> int:
        return self.cache_prefill + self.prefill_len + self.decode_steps

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny-f32", "f32", 256, 8, 2, 768, 256, None, 1e-5, 1e4,
                batch=1, prefill_len=64, decode_steps=16),
    2: Workload(2, "llama7b-block-prefill", "bf16", 4096, 32, 32, 11008, 256, None, 1e-6, 1e4,
                batch=4, prefill_len=2048, decode_steps=0),
    3: Workload(3, "llama3-8b-block-prefill-decode", "bf16", 4096, 32, 8, 14336, 1024, 1.3, 1e-5, 5e5,
                batch=1, prefill_len=8192, decode_steps=128),
    4: Workload(4, "llama2-70b-block-decode", "bf16", 8192, 64, 8, 28672, 1024, 1.3, 1e-5, 1e4,
                batch=32, prefill_len=0, decode_steps=1, cache_prefill=4096),
    5: Workload(5, "llama3-8b-stack", "bf16", 4096, 32, 8, 14336, 1024, 1.3, 1e-5, 5e5,
                batch=64, prefill_len=2048, decode_steps=256, n_layers=32, vocab_size=128256),
}


def _seed(wid: int, layer: int, tid: int) -> int:
    ss = np.random.SeedSequence(BASE_SEED, spawn_key=(wid, layer, tid))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def normal(shape: Tuple[int, ...], std: float, dtype: str, wid: int, layer: int, tid: int) -> torch.Tensor:
    """Seeded N(0, std^2) CPU tensor in the workload dtype (bf16 by RNE from fp32)."""
    g = torch.Generator().manual_seed(_seed(wid, layer, tid))
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch_dtype(dtype))


def tokens(shape: Tuple[int, ...], vocab: int, wid: int, layer: int = 0) -> torch.Tensor:
    g = torch.Generator().manual_seed(_seed(wid, layer, T_TOKENS))
    return torch.randint(0, vocab, shape, generator=g, dtype=torch.int32)


def norm_gain(w: Workload, layer: int, tid: int) -> torch.Tensor:
    """An RMSNorm weight [dim] as the workload's ``norm_gains`` names it."""
    if w.norm_gains == "ones":
        return torch.ones(w.dim, dtype=torch_dtype(w.dtype))
    g = torch.Generator().manual_seed(_seed(w.wid, layer, tid))
    if w.norm_gains == "normal":
        t = 1.0 + 0.2 * torch.randn(w.dim, generator=g, dtype=torch.float32)
    elif w.norm_gains == "pow2":
        t = torch.exp2(torch.randint(-1, 2, (w.dim,), generator=g).to(torch.float32))
    else:
        raise ValueError(f"unknown norm_gains {w.norm_gains!r}")
    return t.to(torch_dtype(w.dtype))


def block_weights(w: Workload, layer: int = 0) -> dict:
    """Linear weights as nn.Linear stores them, [out, in]; norm weights from norm_gain."""
    D, H, Hkv, d, F = w.dim, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn_hidden
    shapes = {
        "wq": ((H * d, D), T_WQ), "wk": ((Hkv * d, D), T_WK), "wv": ((Hkv * d, D), T_WV),
        "wo": ((D, H * d), T_WO), "w1": ((F, D), T_W1), "w2": ((D, F), T_W2), "w3": ((F, D), T_W3),
    }
    out = {k: normal(s, WEIGHT_STD, w.dtype, w.wid, layer, tid) for k, (s, tid) in shapes.items()}
    out["attention_norm"] = norm_gain(w, layer, T_ATTN_NORM)
    out["ffn_norm"] = norm_gain(w, layer, T_FFN_NORM)
    return out


def activations(w: Workload) -> torch.Tensor:
    """x for the whole run: [B, prefill_len + decode_steps, D], N(0,1).

    Row s < prefill_len feeds the prefill call; row prefill_len + t feeds decode step t.
    """
    xp = normal((w.batch, w.prefill_len, w.dim), 1.0, w.dtype, w.wid, 0, T_X_PREFILL)
    xd = normal((w.batch, w.decode_steps, w.dim), 1.0, w.dtype, w.wid, 0, T_X_DECODE)
    return torch.cat([xp, xd], dim=1)


def prefilled_cache(w: Workload, layer: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Cache rows 0..cache_prefill-1 drawn N(0,1), the rest zero: [B, max_seq_len, Hkv, d]."""
    shape = (w.batch, w.cache_prefill, w.n_kv_heads, w.head_dim)
    ck = torch.zeros((w.batch, w.max_seq_len, w.n_kv_heads, w.head_dim), dtype=torch_dtype(w.dtype))
    cv = torch.zeros_like(ck)
    if w.cache_prefill:
        ck[:, :w.cache_prefill] = normal(shape, 1.0, w.dtype, w.wid, layer, T_CACHE_K)
        cv[:, :w.cache_prefill] = normal(shape, 1.0, w.dtype, w.wid, layer, T_CACHE_V)
    return ck, cv


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a (bf16 or f32) tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def stack_tensors(w: Workload):
    """Embedding [vocab, dim], final RMSNorm weight (norm_gain) and output projection [vocab, dim]."""
    emb = normal((w.vocab_size, w.dim), WEIGHT_STD, w.dtype, w.wid, 0, T_EMBED)
    out = normal((w.vocab_size, w.dim), WEIGHT_STD, w.dtype, w.wid, 0, T_OUTPUT)
    return emb, norm_gain(w, 0, T_FINAL_NORM), out


def prompt_tokens(w: Workload) -> torch.Tensor:
    """Random prompt ids [batch, prefill_len], uniform over the vocabulary."""
    return tokens((w.batch, w.prefill_len), w.vocab_size, w.wid)
