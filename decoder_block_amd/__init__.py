"""MI355X (gfx950) LLaMA decoder-block forward pass: HIP kernels behind a C ABI.

``decoder_block_amd._lib`` binds the C entry points of ``libllama_block.so``
under their C names; ``decoder_block_amd.model`` composes them into the
whole-model step (greedy or top-p sampling).  torch is used only for device memory and streams.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LLAMA_BF16, LLAMA_F32, LlamaError, ModelArgs, block_weights, lib, llama_attn_decode_workspace_size,
    llama_block_decode_at, llama_gqa_attn_decode_static, llama_static_scratch_bytes,
    llama_block_forward, llama_block_forward_events, llama_block_workspace_size, llama_embedding, llama_ffn_hidden_dim,
    llama_ffn_workspace_size, llama_gqa_attn_decode, llama_gqa_attn_prefill, llama_linear, llama_lm_head_argmax,
    llama_lm_head_workspace_size, llama_rmsnorm, llama_rope, llama_rope_freqs, llama_sample_top_p, llama_swiglu_ffn,
    status_str,
)
