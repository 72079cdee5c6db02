"""ctypes binding of libllama_block.so: the C entry points under the same names.

Argument marshalling only: every function converts tensors to device pointers
and the current torch stream to a hipStream_t, calls the C function and raises
``LlamaError`` on a non-zero status.  No arithmetic happens here.  The shared
library must have been built (``python -m decoder_block_amd.build``); a missing
library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllama_block.so")

LLAMA_OK = 0
LLAMA_ERR_INVALID_ARG = -1
LLAMA_ERR_UNSUPPORTED = -2
LLAMA_ERR_WORKSPACE_TOO_SMALL = -3
LLAMA_ERR_HIP = -4
LLAMA_ERR_SCRATCH_TOO_SMALL = -5
LLAMA_F32 = 0
LLAMA_BF16 = 1

# every symbol include/llama_block.h declares
EXPORTS = (
    "llama_status_str", "llama_ffn_hidden_dim", "llama_block_workspace_size",
    "llama_attn_decode_workspace_size", "llama_ffn_workspace_size", "llama_rope_freqs",
    "llama_rmsnorm", "llama_rope", "llama_gqa_attn_prefill", "llama_gqa_attn_decode",
    "llama_swiglu_ffn", "llama_linear", "llama_block_forward", "llama_block_forward_events",
    "llama_block_decode_at", "llama_embedding",
    "llama_lm_head_workspace_size", "llama_lm_head_argmax", "llama_sample_top_p",
    "llama_gqa_attn_decode_static", "llama_static_scratch_bytes",
)


class LlamaError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn} returned {status}: {status_str(status)}")


class CModelArgs(ctypes.Structure):
    _fields_ = [
        ("dim", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("vocab_size", ctypes.c_int32), ("multiple_of", ctypes.c_int32),
        ("ffn_dim_multiplier", ctypes.c_float), ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("max_batch_size", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
    ]


class CBlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attention_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w1", "w2", "w3")]


@dataclasses.dataclass
class ModelArgs:
    """Mirror of the C struct (and of the pages' ModelArgs plus rope_theta)."""
    dim: int = 4096
    n_layers: int = 32
    n_heads: int = 32
    n_kv_heads: Optional[int] = None
    vocab_size: int = -1
    multiple_of: int = 256
    ffn_dim_multiplier: Optional[float] = None
    norm_eps: float = 1e-5
    rope_theta: float = 10000.0
    max_batch_size: int = 32
    max_seq_len: int = 2048

    def c(self) -> CModelArgs:
        return CModelArgs(self.dim, self.n_layers, self.n_heads, self.n_kv_heads or 0, self.vocab_size,
                          self.multiple_of, self.ffn_dim_multiplier or 0.0, self.norm_eps, self.rope_theta,
                          self.max_batch_size, self.max_seq_len)


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decoder_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        A = ctypes.POINTER(CModelArgs)
        sig = {
            "llama_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "llama_ffn_hidden_dim": ([A, ctypes.POINTER(I32)], ctypes.c_int),
            "llama_block_workspace_size": ([A, I32, I32, I32, ctypes.c_int, ctypes.POINTER(SZ)], ctypes.c_int),
            "llama_attn_decode_workspace_size": ([A, I32, I32, ctypes.POINTER(SZ)], ctypes.c_int),
            "llama_ffn_workspace_size": ([I64, I32, I32, ctypes.c_int, ctypes.POINTER(SZ)], ctypes.c_int),
            "llama_lm_head_workspace_size": ([I32, I32, I32, ctypes.c_int, ctypes.POINTER(SZ)], ctypes.c_int),
            "llama_rope_freqs": ([P, I32, I32, F, P], ctypes.c_int),
            "llama_rmsnorm": ([P, P, P, I64, I32, F, ctypes.c_int, P], ctypes.c_int),
            "llama_rope": ([P, P, P, I32, I32, I32, I32, I32, I32, I32, ctypes.c_int, P], ctypes.c_int),
            "llama_gqa_attn_prefill": ([P, P, P, P, P, P, A, I32, I32, I32, ctypes.c_int, P], ctypes.c_int),
            "llama_gqa_attn_decode": ([P, P, P, P, P, P, A, I32, I32, P, SZ, ctypes.c_int, P], ctypes.c_int),
            "llama_swiglu_ffn": ([P, P, P, P, P, I64, I32, I32, P, SZ, ctypes.c_int, P], ctypes.c_int),
            "llama_linear": ([P, P, P, I64, I32, I32, ctypes.c_int, P], ctypes.c_int),
            "llama_block_forward": ([A, ctypes.POINTER(CBlockWeights), P, P, P, I32, P, P, I32, I32, I32, P, SZ,
                                     ctypes.c_int, P], ctypes.c_int),
            "llama_block_forward_events": ([A, ctypes.POINTER(CBlockWeights), P, P, P, I32, P, P, I32, I32, I32, P,
                                            SZ, ctypes.c_int, P, ctypes.POINTER(P)], ctypes.c_int),
            "llama_block_decode_at": ([A, ctypes.POINTER(CBlockWeights), P, P, P, I32, P, P, I32, P, I32, P, SZ,
                                       ctypes.c_int, P], ctypes.c_int),
            "llama_embedding": ([P, P, P, I64, I32, I32, ctypes.c_int, P], ctypes.c_int),
            "llama_lm_head_argmax": ([P, I64, P, P, P, P, I32, I32, I32, F, P, SZ, ctypes.c_int, P], ctypes.c_int),
            "llama_sample_top_p": ([P, P, I32, I32, F, F, P, P], ctypes.c_int),
            "llama_gqa_attn_decode_static": ([P, P, P, P, P, P, A, I32, I32, ctypes.c_int, P], ctypes.c_int),
            "llama_static_scratch_bytes": ([], SZ),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().llama_status_str(status).decode()


def _check(status: int, fn: str) -> None:
    if status != LLAMA_OK:
        raise LlamaError(status, fn)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return LLAMA_BF16
    if t.dtype == torch.float32:
        return LLAMA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ host helpers
def llama_ffn_hidden_dim(args: ModelArgs) -> int:
    out = ctypes.c_int32()
    _check(lib().llama_ffn_hidden_dim(ctypes.byref(args.c()), ctypes.byref(out)), "llama_ffn_hidden_dim")
    return out.value


def llama_block_workspace_size(args: ModelArgs, bsz: int, seqlen: int, start_pos: int, dtype: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().llama_block_workspace_size(ctypes.byref(args.c()), bsz, seqlen, start_pos, dtype,
                                            ctypes.byref(out)), "llama_block_workspace_size")
    return out.value


def llama_attn_decode_workspace_size(args: ModelArgs, bsz: int, start_pos: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().llama_attn_decode_workspace_size(ctypes.byref(args.c()), bsz, start_pos, ctypes.byref(out)),
           "llama_attn_decode_workspace_size")
    return out.value


def llama_ffn_workspace_size(rows: int, dim: int, hidden: int, dtype: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().llama_ffn_workspace_size(rows, dim, hidden, dtype, ctypes.byref(out)), "llama_ffn_workspace_size")
    return out.value


def llama_lm_head_workspace_size(bsz: int, dim: int, vocab: int, dtype: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().llama_lm_head_workspace_size(bsz, dim, vocab, dtype, ctypes.byref(out)),
           "llama_lm_head_workspace_size")
    return out.value


# ------------------------------------------------------------------ device entry points
def llama_rope_freqs(freqs, head_dim: int, end: int, rope_theta: float, stream=None) -> None:
    _check(lib().llama_rope_freqs(_ptr(freqs), head_dim, end, rope_theta, _stream(stream)), "llama_rope_freqs")


def llama_rmsnorm(x, w, y, rows: int, dim: int, eps: float, stream=None) -> None:
    _check(lib().llama_rmsnorm(_ptr(x), _ptr(w), _ptr(y), rows, dim, eps, _dtype(x), _stream(stream)),
           "llama_rmsnorm")


def llama_rope(xq, xk, freqs, freqs_end: int, bsz: int, seqlen: int, start_pos: int, n_heads: int,
               n_kv_heads: int, head_dim: int, stream=None) -> None:
    _check(lib().llama_rope(_ptr(xq), _ptr(xk), _ptr(freqs), freqs_end, bsz, seqlen, start_pos, n_heads,
                            n_kv_heads, head_dim, _dtype(xq), _stream(stream)), "llama_rope")


def llama_gqa_attn_prefill(xq, xk, xv, cache_k, cache_v, out, args: ModelArgs, bsz: int, seqlen: int,
                           start_pos: int, stream=None) -> None:
    _check(lib().llama_gqa_attn_prefill(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(cache_k), _ptr(cache_v), _ptr(out),
                                        ctypes.byref(args.c()), bsz, seqlen, start_pos, _dtype(xq),
                                        _stream(stream)), "llama_gqa_attn_prefill")


def llama_gqa_attn_decode(xq, xk, xv, cache_k, cache_v, out, args: ModelArgs, bsz: int, start_pos: int, ws,
                          ws_bytes: int, stream=None) -> None:
    _check(lib().llama_gqa_attn_decode(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(cache_k), _ptr(cache_v), _ptr(out),
                                       ctypes.byref(args.c()), bsz, start_pos, _ptr(ws), ws_bytes, _dtype(xq),
                                       _stream(stream)), "llama_gqa_attn_decode")


def llama_gqa_attn_decode_static(xq, xk, xv, cache_k, cache_v, out, args: ModelArgs, bsz: int, start_pos: int,
                                 stream=None) -> None:
    """llama_gqa_attn_decode without a workspace: the partials go to the library's static
    per-GPU scratch array (no allocation on the call)."""
    _check(lib().llama_gqa_attn_decode_static(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(cache_k), _ptr(cache_v),
                                              _ptr(out), ctypes.byref(args.c()), bsz, start_pos, _dtype(xq),
                                              _stream(stream)), "llama_gqa_attn_decode_static")


def llama_static_scratch_bytes() -> int:
    return int(lib().llama_static_scratch_bytes())


def llama_swiglu_ffn(x, w1, w3, w2, y, rows: int, dim: int, hidden: int, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().llama_swiglu_ffn(_ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y), rows, dim, hidden, _ptr(ws),
                                  ws_bytes, _dtype(x), _stream(stream)), "llama_swiglu_ffn")


def llama_linear(x, w, y, rows: int, in_features: int, out_features: int, stream=None) -> None:
    _check(lib().llama_linear(_ptr(x), _ptr(w), _ptr(y), rows, in_features, out_features, _dtype(x),
                              _stream(stream)), "llama_linear")


BLOCK_TENSORS = ("attention_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w1", "w2", "w3")


def block_tensor_shapes(args: ModelArgs) -> dict:
    """The [out, in] (or [dim]) shape of each block parameter that ``args`` implies."""
    D, H = args.dim, args.n_heads
    Hkv = args.n_kv_heads or H
    d = D // H
    F = llama_ffn_hidden_dim(args)
    return {"attention_norm": (D,), "ffn_norm": (D,), "wq": (H * d, D), "wk": (Hkv * d, D), "wv": (Hkv * d, D),
            "wo": (D, H * d), "w1": (F, D), "w3": (F, D), "w2": (D, F)}


def check_block_tensors(args: ModelArgs, weights, cache_k, cache_v, x, out, bsz: int, seqlen: int) -> None:
    """The C ABI receives bare pointers and derives every extent from ``args``.  When
    the caller passes tensors, their shapes are checked here, on the host, before a
    kernel could read or write past them: each weight against the shape ``args``
    implies (the FFN width from dim, multiple_of and ffn_dim_multiplier), the caches
    against [max_batch_size, max_seq_len, n_kv_heads, head_dim], x and out against
    bsz * seqlen rows of dim.  Raw pointers (ints) are passed through unchecked."""
    def numel(t):
        return None if t is None or isinstance(t, int) else t.numel()
    if isinstance(weights, dict):
        for name, shape in block_tensor_shapes(args).items():
            t = weights[name]
            if not isinstance(t, int) and tuple(t.shape) != shape:
                raise ValueError(f"weight {name} has shape {tuple(t.shape)}; the model arguments imply {shape}")
    Hkv = args.n_kv_heads or args.n_heads
    cache = args.max_batch_size * args.max_seq_len * Hkv * (args.dim // args.n_heads)
    for name, t in (("cache_k", cache_k), ("cache_v", cache_v)):
        n = numel(t)
        if n is not None and n < cache:
            raise ValueError(f"{name} holds {n} elements; max_batch_size x max_seq_len x n_kv_heads x head_dim "
                             f"is {cache}")
    act = bsz * seqlen * args.dim
    for name, t in (("x", x), ("out", out)):
        n = numel(t)
        if n is not None and n < act:
            raise ValueError(f"{name} holds {n} elements; bsz x seqlen x dim is {act}")


def block_weights(tensors: dict) -> CBlockWeights:
    return CBlockWeights(*[_ptr(tensors[n]) for n in BLOCK_TENSORS])


def llama_block_forward(args: ModelArgs, weights, cache_k, cache_v, freqs, freqs_end: int, x, out, bsz: int,
                        seqlen: int, start_pos: int, ws, ws_bytes: int, stream=None) -> None:
    check_block_tensors(args, weights, cache_k, cache_v, x, out, bsz, seqlen)
    w = weights if isinstance(weights, CBlockWeights) else block_weights(weights)
    _check(lib().llama_block_forward(ctypes.byref(args.c()), ctypes.byref(w), _ptr(cache_k), _ptr(cache_v),
                                     _ptr(freqs), freqs_end, _ptr(x), _ptr(out), bsz, seqlen, start_pos, _ptr(ws),
                                     ws_bytes, _dtype(x), _stream(stream)), "llama_block_forward")


def llama_block_decode_at(args: ModelArgs, weights, cache_k, cache_v, freqs, freqs_end: int, x, out, bsz: int,
                          start_pos_dev, max_start_pos: int, ws, ws_bytes: int, stream=None) -> None:
    """One-token block decode at the position held in ``start_pos_dev`` (device int32)."""
    check_block_tensors(args, weights, cache_k, cache_v, x, out, bsz, 1)
    w = weights if isinstance(weights, CBlockWeights) else block_weights(weights)
    _check(lib().llama_block_decode_at(ctypes.byref(args.c()), ctypes.byref(w), _ptr(cache_k), _ptr(cache_v),
                                       _ptr(freqs), freqs_end, _ptr(x), _ptr(out), bsz, _ptr(start_pos_dev),
                                       max_start_pos, _ptr(ws), ws_bytes, _dtype(x), _stream(stream)),
           "llama_block_decode_at")


def llama_block_forward_events(args: ModelArgs, weights, cache_k, cache_v, freqs, freqs_end: int, x, out, bsz: int,
                               seqlen: int, start_pos: int, ws, ws_bytes: int, events, stream=None) -> None:
    """``events``: 8 torch.cuda.Event(enable_timing=True) (or raw hipEvent_t handles)."""
    check_block_tensors(args, weights, cache_k, cache_v, x, out, bsz, seqlen)
    w = weights if isinstance(weights, CBlockWeights) else block_weights(weights)
    st = _stream(stream)
    handles = []
    for e in events:
        if isinstance(e, int):
            handles.append(e)
        else:
            if not e.cuda_event:
                e.record()  # torch creates the HIP event on first use
            handles.append(e.cuda_event)
    arr = (ctypes.c_void_p * 8)(*handles)
    _check(lib().llama_block_forward_events(ctypes.byref(args.c()), ctypes.byref(w), _ptr(cache_k), _ptr(cache_v),
                                            _ptr(freqs), freqs_end, _ptr(x), _ptr(out), bsz, seqlen, start_pos,
                                            _ptr(ws), ws_bytes, _dtype(x), st, arr), "llama_block_forward_events")


def llama_embedding(tokens, table, out, n: int, dim: int, vocab: int, stream=None) -> None:
    _check(lib().llama_embedding(_ptr(tokens), _ptr(table), _ptr(out), n, dim, vocab, _dtype(table),
                                 _stream(stream)), "llama_embedding")


def llama_lm_head_argmax(h, h_row_stride: int, norm_w, w_out, logits, next_tok, bsz: int, dim: int, vocab: int,
                         eps: float, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().llama_lm_head_argmax(_ptr(h), h_row_stride, _ptr(norm_w), _ptr(w_out), _ptr(logits),
                                      _ptr(next_tok), bsz, dim, vocab, eps, _ptr(ws), ws_bytes, _dtype(h),
                                      _stream(stream)), "llama_lm_head_argmax")


def llama_sample_top_p(logits, next_tok, bsz: int, vocab: int, temperature: float, top_p: float, uniforms=None,
                       stream=None) -> None:
    _check(lib().llama_sample_top_p(_ptr(logits), _ptr(next_tok), bsz, vocab, temperature, top_p,
                                    _ptr(uniforms) if uniforms is not None else None, _stream(stream)),
           "llama_sample_top_p")
