"""Device-side state for running one decoder block through the C ABI.

Holds the block's weights, KV cache, RoPE table and a workspace on the GPU
(torch allocates; the library allocates nothing) and calls
``llama_block_forward`` on the current stream.  Every step of the forward pass
runs in the HIP library.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import _lib as L


def check_weight_shapes(args: L.ModelArgs, weights: Dict[str, torch.Tensor]) -> None:
    """The C ABI receives bare pointers and derives every extent from ``args`` (the
    FFN width from dim, multiple_of and ffn_dim_multiplier): weights of another shape
    would be read out of bounds, so their shapes are checked here, on the host."""
    for name, shape in L.block_tensor_shapes(args).items():
        got = tuple(weights[name].shape)
        if got != shape:
            raise ValueError(f"weight {name} has shape {got}; the model arguments imply {shape}")


class BlockRunner:
    def __init__(self, args: L.ModelArgs, weights: Dict[str, torch.Tensor], dtype: torch.dtype,
                 device="cuda:0", cache=None, share_freqs=None):
        self.args = args
        self.dtype = dtype
        self.ldt = L.LLAMA_BF16 if dtype == torch.bfloat16 else L.LLAMA_F32
        self.device = torch.device(device)
        self.head_dim = args.dim // args.n_heads
        n_kv = args.n_kv_heads or args.n_heads
        check_weight_shapes(args, weights)
        self.w = {k: v.to(self.device, dtype) for k, v in weights.items()}
        self.cw = L.block_weights(self.w)
        if cache is None:
            shape = (args.max_batch_size, args.max_seq_len, n_kv, self.head_dim)
            self.cache_k = torch.zeros(shape, dtype=dtype, device=self.device)
            self.cache_v = torch.zeros(shape, dtype=dtype, device=self.device)
        else:
            self.cache_k, self.cache_v = (c.to(self.device, dtype) for c in cache)
        if share_freqs is not None:
            self.freqs, self.freqs_end = share_freqs
        else:
            # the table spans 2 * max_seq_len positions, as precompute_freqs_cis is called
            self.freqs_end = 2 * args.max_seq_len
            self.freqs = torch.empty(self.freqs_end, self.head_dim // 2, 2, dtype=torch.float32,
                                     device=self.device)
            L.llama_rope_freqs(self.freqs, self.head_dim, self.freqs_end, args.rope_theta)
        self.ws: Optional[torch.Tensor] = None

    def workspace(self, bsz: int, seqlen: int, start_pos: int) -> int:
        need = L.llama_block_workspace_size(self.args, bsz, seqlen, start_pos, self.ldt)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return need

    def reserve(self, bsz: int, seqlen: int, start_pos: int) -> None:
        """Grow the workspace ahead of a timed loop."""
        self.workspace(bsz, seqlen, start_pos)

    def forward(self, x: torch.Tensor, start_pos: int, out: Optional[torch.Tensor] = None,
                events=None) -> torch.Tensor:
        bsz, seqlen, _ = x.shape
        need = self.workspace(bsz, seqlen, start_pos)
        if out is None:
            out = torch.empty_like(x)
        if events is None:
            L.llama_block_forward(self.args, self.cw, self.cache_k, self.cache_v, self.freqs, self.freqs_end, x, out,
                                  bsz, seqlen, start_pos, self.ws, self.ws.numel())
        else:
            L.llama_block_forward_events(self.args, self.cw, self.cache_k, self.cache_v, self.freqs, self.freqs_end,
                                         x, out, bsz, seqlen, start_pos, self.ws, self.ws.numel(), events)
        del need
        return out


def model_args_for(w, max_batch: Optional[int] = None, max_seq: Optional[int] = None) -> L.ModelArgs:
    """ModelArgs of a ``workloads.Workload``."""
    return L.ModelArgs(dim=w.dim, n_layers=w.n_layers, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads,
                       vocab_size=w.vocab_size or -1, multiple_of=w.multiple_of,
                       ffn_dim_multiplier=w.ffn_dim_multiplier, norm_eps=w.norm_eps, rope_theta=w.rope_theta,
                       max_batch_size=max_batch or w.batch, max_seq_len=max_seq or w.max_seq_len)
