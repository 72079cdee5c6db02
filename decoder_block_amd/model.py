"""Whole-model generation on one GPU through the C ABI.

Token embedding -> n_layers x llama_block_forward -> final RMSNorm + output
projection of the last position -> argmax or top-p sampling, with the token
written on the device and fed straight back as the next call's input (no host
round trip per token).  Follows the linkmax.top walkthrough of Meta's LLaMA code,
section 3.2.2 (Transformer.forward: embedding, layers, norm, output on the last
position) and section 3.3 (generate: one prefill call, then one-token calls at
the previous position; argmax when the temperature is 0, else softmax at the
temperature and sample_top_p).

torch only allocates device memory and provides the stream; every step of the
forward pass runs in the HIP library.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional

import torch

from . import _lib as L
from .runner import BlockRunner


class StackRunner:
    def __init__(self, args: L.ModelArgs, layer_weights: Callable[[int], Dict[str, torch.Tensor]],
                 embedding: torch.Tensor, norm_w: torch.Tensor, w_out: torch.Tensor, dtype=torch.bfloat16,
                 device="cuda:0"):
        """``layer_weights(l)`` returns layer l's tensors (CPU or device); they are moved
        to the device one layer at a time."""
        self.args = args
        self.dtype = dtype
        self.ldt = L.LLAMA_BF16 if dtype == torch.bfloat16 else L.LLAMA_F32
        self.device = torch.device(device)
        self.layers: List[BlockRunner] = []
        freqs = None
        for l in range(args.n_layers):
            r = BlockRunner(args, layer_weights(l), dtype, self.device, share_freqs=freqs)
            freqs = (r.freqs, r.freqs_end)
            self.layers.append(r)
        self.embedding = embedding.to(self.device, dtype)
        self.norm_w = norm_w.to(self.device, dtype)
        self.w_out = w_out.to(self.device, dtype)
        self.vocab = self.w_out.shape[0]
        self.ws: Optional[torch.Tensor] = None
        self.bufs: Optional[List[torch.Tensor]] = None

    def _workspace(self, bsz: int, seqlen: int, start_pos: int) -> int:
        need = L.llama_block_workspace_size(self.args, bsz, seqlen, start_pos, self.ldt)
        need = max(need, L.llama_lm_head_workspace_size(bsz, self.args.dim, self.vocab, self.ldt))
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.ws.numel()

    def _acts(self, bsz: int, seqlen: int) -> List[torch.Tensor]:
        n = bsz * seqlen * self.args.dim
        if self.bufs is None or self.bufs[0].numel() < n:
            self.bufs = [torch.empty(n, dtype=self.dtype, device=self.device) for _ in range(2)]
        return [b[:n].view(bsz, seqlen, self.args.dim) for b in self.bufs]

    def forward(self, tokens: torch.Tensor, start_pos: int, logits: torch.Tensor, next_tok: torch.Tensor,
                layer_hook=None, layer_events=None) -> None:
        """One call (prefill when tokens has several columns, decode when one):
        writes the last position's fp32 logits [bsz, vocab] and greedy ids [bsz].
        ``layer_events`` (optional): one list of 8 timing events per layer, recorded
        between the block's stages as llama_block_forward_events describes."""
        bsz, seqlen = tokens.shape
        ws_bytes = self._workspace(bsz, seqlen, start_pos)
        a, b = self._acts(bsz, seqlen)
        D = self.args.dim
        L.llama_embedding(tokens, self.embedding, a, bsz * seqlen, D, self.vocab)
        for i, layer in enumerate(self.layers):
            if layer_events is not None:
                L.llama_block_forward_events(self.args, layer.cw, layer.cache_k, layer.cache_v, layer.freqs,
                                             layer.freqs_end, a, b, bsz, seqlen, start_pos, self.ws, ws_bytes,
                                             layer_events[i])
            else:
                L.llama_block_forward(self.args, layer.cw, layer.cache_k, layer.cache_v, layer.freqs,
                                      layer.freqs_end, a, b, bsz, seqlen, start_pos, self.ws, ws_bytes)
            if layer_hook is not None:
                layer_hook(i, a, b)
            a, b = b, a
        last = a[:, seqlen - 1]                # row stride seqlen * dim
        L.llama_lm_head_argmax(last, seqlen * D, self.norm_w, self.w_out, logits, next_tok, bsz, D, self.vocab,
                               self.args.norm_eps, self.ws, ws_bytes)

    def decode_step_at(self, tok: torch.Tensor, pos_dev: torch.Tensor, max_pos: int, logits: torch.Tensor,
                       temperature: float = 0.0, top_p: float = 0.95, u: Optional[torch.Tensor] = None) -> None:
        """One-token step at the position held on the device in ``pos_dev`` (int32 [1],
        at most ``max_pos``): reads the ids in ``tok`` [bsz], overwrites them with the
        chosen ids (argmax, or top-p with the uniforms in ``u`` [bsz] when the
        temperature is positive) and advances ``pos_dev`` by one.  Every argument is
        a fixed buffer and nothing is allocated once the workspace exists, so the
        step can be captured in a HIP graph once and replayed position after
        position."""
        bsz = tok.shape[0]
        ws_bytes = self._workspace(bsz, 1, max_pos)
        a, b = self._acts(bsz, 1)
        D = self.args.dim
        L.llama_embedding(tok, self.embedding, a, bsz, D, self.vocab)
        for layer in self.layers:
            L.llama_block_decode_at(self.args, layer.cw, layer.cache_k, layer.cache_v, layer.freqs, layer.freqs_end,
                                    a, b, bsz, pos_dev, max_pos, self.ws, ws_bytes)
            a, b = b, a
        L.llama_lm_head_argmax(a[:, 0], D, self.norm_w, self.w_out, logits, tok, bsz, D, self.vocab,
                               self.args.norm_eps, self.ws, ws_bytes)
        if temperature > 0:
            L.llama_sample_top_p(logits, tok, bsz, self.vocab, temperature, top_p, u)
        pos_dev.add_(1)

    def generate(self, prompt: torch.Tensor, steps: int, on_step=None, temperature: float = 0.0,
                 top_p: float = 0.95, uniforms: Optional[torch.Tensor] = None, graph: bool = False) -> torch.Tensor:
        """Generation: prefill the prompt, then ``steps`` one-token calls.
        Returns the generated ids [steps + 1, bsz]: row t is chosen on the device
        from call t's logits and is passed, as is, as the input ids of call t + 1
        (no host synchronisation inside the loop).  temperature 0 takes the argmax;
        a positive temperature samples with the nucleus cut top_p, call t drawing
        with uniforms[t] ([steps + 1, bsz] floats in [0, 1), on the device).

        graph=True runs the first one-token call eagerly, captures the next one
        (embedding, every layer, final norm, output projection, token choice and
        position advance) in a HIP graph and replays it for the rest; the position
        lives on the device, and between replays only the chosen ids (and the
        next uniforms) are copied on the device.  The results are those of
        graph=False."""
        bsz, S = prompt.shape
        out = torch.empty(steps + 1, bsz, dtype=torch.int32, device=self.device)
        logits = torch.empty(bsz, self.vocab, dtype=torch.float32, device=self.device)
        sampled = temperature > 0
        if sampled and (uniforms is None or tuple(uniforms.shape) != (steps + 1, bsz)):
            raise ValueError("sampling needs uniforms of shape [steps + 1, bsz] on the device")

        def pick(t):
            if sampled:
                L.llama_sample_top_p(logits, out[t], bsz, self.vocab, temperature, top_p, uniforms[t])
            if on_step is not None:
                on_step(t, logits, out[t])
        self.forward(prompt, 0, logits, out[0])
        pick(0)
        if not graph:
            for t in range(steps):
                self.forward(out[t].view(bsz, 1), S + t, logits, out[t + 1])
                pick(t + 1)
            return out
        if steps == 0:
            return out
        max_pos = S + steps - 1
        tok = out[0].clone()
        pos = torch.full((1,), S, dtype=torch.int32, device=self.device)
        u = torch.empty(bsz, dtype=torch.float32, device=self.device) if sampled else None

        def run_step(t, replay):
            if sampled:
                u.copy_(uniforms[t])
            if replay is None:
                self.decode_step_at(tok, pos, max_pos, logits, temperature, top_p, u)
            else:
                replay.replay()
            out[t].copy_(tok)
            if on_step is not None:
                on_step(t, logits, out[t])
        run_step(1, None)                      # eager: also loads every kernel before the capture
        if steps > 1:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.decode_step_at(tok, pos, max_pos, logits, temperature, top_p, u)
            for t in range(2, steps + 1):
                run_step(t, g)
        return out
