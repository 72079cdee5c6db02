"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-only helpers and argument validation behave as documented.  No call here
reaches a kernel launch (every device call below fails validation first)."""
import ctypes
import os
import re

import pytest

import decoder_block_amd as dba
from decoder_block_amd import _lib as L
from oracle import block as ob
import workloads as wl

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "llama_block.h")


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(llama_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = dba.lib()
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.EXPORTS) == names


def args_for(w: wl.Workload, **kw):
    a = dba.ModelArgs(dim=w.dim, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, multiple_of=w.multiple_of,
                      ffn_dim_multiplier=w.ffn_dim_multiplier, norm_eps=w.norm_eps, rope_theta=w.rope_theta,
                      max_batch_size=w.batch, max_seq_len=max(w.max_seq_len, 1))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_ffn_hidden_dim_matches_oracle_and_workloads():
    for w in wl.WORKLOADS.values():
        assert dba.llama_ffn_hidden_dim(args_for(w)) == w.ffn_hidden
        assert ob.ffn_hidden_dim(w.dim, w.multiple_of, w.ffn_dim_multiplier) == w.ffn_hidden
    for dim in (64, 256, 1000, 5120, 6656, 8192):
        for mo in (1, 32, 256):
            for mult in (None, 1.3, 2.0):
                a = dba.ModelArgs(dim=dim, n_heads=1, multiple_of=mo, ffn_dim_multiplier=mult)
                # float multiplier at the ABI: compare with the oracle fed the same float32 value
                m32 = None if mult is None else float(ctypes.c_float(mult).value)
                assert dba.llama_ffn_hidden_dim(a) == ob.ffn_hidden_dim(dim, mo, m32)


def test_status_strings():
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(dba.status_str(s), str) and dba.status_str(s)


def test_workspace_sizes_cover_the_intermediates():
    w = wl.WORKLOADS[3]
    a = args_for(w)
    n = w.prefill_len
    need = dba.llama_block_workspace_size(a, 1, n, 0, dba.LLAMA_BF16)
    D, F = w.dim, w.ffn_hidden
    assert need >= 2 * n * (4 * D + F)  # xn, q, o, h, hn (H*d = D) and the gated activation
    dec = dba.llama_block_workspace_size(a, 1, 1, n, dba.LLAMA_BF16)
    assert dec >= dba.llama_attn_decode_workspace_size(a, 1, n)
    with pytest.raises(dba.LlamaError):
        dba.llama_block_workspace_size(a, 2, 1, 0, dba.LLAMA_BF16)   # bsz > max_batch_size
    with pytest.raises(dba.LlamaError):
        dba.llama_block_workspace_size(a, 1, w.max_seq_len + 1, 0, dba.LLAMA_BF16)


def _raw_block_forward(a, **over):
    """Call llama_block_forward through ctypes with dummy non-null pointers."""
    lib = dba.lib()
    fake = 1 << 20                       # 16-byte aligned, never dereferenced: validation fails first
    kw = dict(bsz=1, seqlen=4, start_pos=0, freqs_end=16, ws_bytes=0, dtype=dba.LLAMA_BF16, weights=None,
              x=fake, out=fake * 2, ck=fake, cv=fake, freqs=fake, ws=fake)
    kw.update(over)
    w = kw["weights"] or L.CBlockWeights(*([fake] * 9))
    return lib.llama_block_forward(ctypes.byref(a.c()), ctypes.byref(w), kw["ck"], kw["cv"], kw["freqs"],
                                   kw["freqs_end"], kw["x"], kw["out"], kw["bsz"], kw["seqlen"], kw["start_pos"],
                                   kw["ws"], kw["ws_bytes"], kw["dtype"], None)


def test_block_forward_validation_errors():
    a = dba.ModelArgs(dim=256, n_heads=2, n_kv_heads=1, max_batch_size=2, max_seq_len=16)
    E, U, W = dba._lib.LLAMA_ERR_INVALID_ARG, dba._lib.LLAMA_ERR_UNSUPPORTED, dba._lib.LLAMA_ERR_WORKSPACE_TOO_SMALL
    assert _raw_block_forward(a) == W                       # valid call, workspace missing
    assert _raw_block_forward(a, bsz=3) == E                 # bsz > max_batch_size
    assert _raw_block_forward(a, bsz=0) == E
    assert _raw_block_forward(a, seqlen=0) == E
    assert _raw_block_forward(a, start_pos=-1) == E
    assert _raw_block_forward(a, start_pos=13) == E          # start_pos + seqlen > max_seq_len
    assert _raw_block_forward(a, freqs_end=3) == E           # RoPE table too short
    assert _raw_block_forward(a, x=None) == E
    assert _raw_block_forward(a, ck=None) == E
    assert _raw_block_forward(a, out=(1 << 20) + 64) == E    # out overlaps x
    assert _raw_block_forward(a, x=(1 << 20) + 2) == E       # misaligned
    assert _raw_block_forward(a, dtype=7) == E
    bad = L.CBlockWeights(*([1 << 20] * 8 + [None]))
    assert _raw_block_forward(a, weights=bad) == E
    assert _raw_block_forward(dba.ModelArgs(dim=256, n_heads=3, max_batch_size=2, max_seq_len=16)) == E  # dim % H
    assert _raw_block_forward(dba.ModelArgs(dim=256, n_heads=4, n_kv_heads=3, max_batch_size=2,
                                            max_seq_len=16)) == E                    # H % Hkv
    assert _raw_block_forward(dba.ModelArgs(dim=256, n_heads=8, max_batch_size=2, max_seq_len=16)) == U  # d=32 bf16
    assert _raw_block_forward(dba.ModelArgs(dim=256, n_heads=8, max_batch_size=2, max_seq_len=16),
                              dtype=dba.LLAMA_F32) == W                             # d=32 is built for f32
    # one sequence's cache rows (max_seq_len * n_kv_heads * head_dim) must stay below 2^31 elements
    assert _raw_block_forward(dba.ModelArgs(dim=8192, n_heads=64, n_kv_heads=64, max_batch_size=1,
                                            max_seq_len=1 << 18)) == U
    assert _raw_block_forward(dba.ModelArgs(dim=8192, n_heads=64, n_kv_heads=8, max_batch_size=1,
                                            max_seq_len=1 << 18)) == W


def test_device_entry_points_reject_bad_arguments():
    lib = dba.lib()
    E = dba._lib.LLAMA_ERR_INVALID_ARG
    p = 1 << 20
    assert lib.llama_rmsnorm(None, p, p, 4, 256, 1e-5, dba.LLAMA_BF16, None) == E
    assert lib.llama_rmsnorm(p, p, p, 4, 250, 1e-5, dba.LLAMA_BF16, None) == E       # dim % 8
    assert lib.llama_rmsnorm(p, p, p, -1, 256, 1e-5, dba.LLAMA_BF16, None) == E
    assert lib.llama_rmsnorm(None, None, None, 0, 256, 1e-5, dba.LLAMA_BF16, None) == 0  # empty: no-op
    assert lib.llama_rope(p, p, p, 8, 1, 9, 0, 4, 4, 64, dba.LLAMA_BF16, None) == E     # table too short
    assert lib.llama_rope(p, p, p, 64, 1, 9, 0, 4, 4, 66, dba.LLAMA_BF16, None) == E    # head_dim % 4
    assert lib.llama_rope_freqs(None, 64, 10, 1e4, None) == E
    assert lib.llama_rope_freqs(p, 63, 10, 1e4, None) == E
    assert lib.llama_linear(p, p, p, 4, 100, 64, dba.LLAMA_BF16, None) == E            # in % 8
    assert lib.llama_linear(p, p, p, 4, 128, 66, dba.LLAMA_BF16, None) == E            # out % 4
    assert lib.llama_linear(None, None, None, 0, 128, 64, dba.LLAMA_BF16, None) == 0   # empty
    a = dba.ModelArgs(dim=512, n_heads=4, n_kv_heads=2, max_batch_size=2, max_seq_len=8)
    c = ctypes.byref(a.c())
    assert lib.llama_gqa_attn_prefill(p, p, p, p, p, p, c, 1, 9, 0, dba.LLAMA_BF16, None) == E
    assert lib.llama_gqa_attn_prefill(p, None, p, p, p, p, c, 1, 4, 0, dba.LLAMA_BF16, None) == E
    assert lib.llama_gqa_attn_decode(p, p, p, p, p, p, c, 1, 8, p, 1 << 30, dba.LLAMA_BF16, None) == E
    assert lib.llama_gqa_attn_decode(p, p, p, p, p, p, c, 3, 5, p, 1 << 30, dba.LLAMA_BF16, None) == E
    big = dba.ModelArgs(dim=8192, n_heads=64, n_kv_heads=8, max_batch_size=1, max_seq_len=9000)
    assert dba.llama_attn_decode_workspace_size(big, 1, 8000) > 0
    assert lib.llama_gqa_attn_decode(p, p, p, p, p, p, ctypes.byref(big.c()), 1, 8000, p, 16, dba.LLAMA_BF16,
                                     None) == dba._lib.LLAMA_ERR_WORKSPACE_TOO_SMALL
    assert lib.llama_swiglu_ffn(p, p, p, p, p, 4, 256, 768, p, 0, dba.LLAMA_BF16, None) == \
        dba._lib.LLAMA_ERR_WORKSPACE_TOO_SMALL
    assert lib.llama_embedding(p, p, p, 4, 250, 10, dba.LLAMA_BF16, None) == E
    assert lib.llama_sample_top_p(None, p, 4, 100, 0.8, 0.9, p, None) == E             # no logits
    assert lib.llama_sample_top_p(p, p, 0, 100, 0.8, 0.9, p, None) == E                # bsz < 1
    assert lib.llama_sample_top_p(p, p, 4, 0, 0.8, 0.9, p, None) == E                  # vocab < 1
    assert lib.llama_sample_top_p(p, p, 4, 100, 0.8, float("nan"), p, None) == E       # top_p NaN
    assert lib.llama_sample_top_p(p, p, 4, 100, float("nan"), 0.9, p, None) == E       # temperature NaN
    assert lib.llama_sample_top_p(p, p, 4, 100, 0.8, 0.9, None, None) == E             # sampling needs uniforms
    assert lib.llama_lm_head_argmax(p, 100, p, p, p, p, 2, 256, 1000, 1e-5, p, 1 << 30, dba.LLAMA_BF16, None) == E


def _raw_decode_at(a, **over):
    """Call llama_block_decode_at through ctypes with dummy non-null pointers."""
    lib = dba.lib()
    fake = 1 << 20
    kw = dict(bsz=1, pos=fake * 4, max_pos=0, freqs_end=16, ws_bytes=0, dtype=dba.LLAMA_BF16, x=fake,
              out=fake * 2, ck=fake, cv=fake, freqs=fake, ws=fake)
    kw.update(over)
    w = L.CBlockWeights(*([fake] * 9))
    return lib.llama_block_decode_at(ctypes.byref(a.c()), ctypes.byref(w), kw["ck"], kw["cv"], kw["freqs"],
                                     kw["freqs_end"], kw["x"], kw["out"], kw["bsz"], kw["pos"], kw["max_pos"],
                                     kw["ws"], kw["ws_bytes"], kw["dtype"], None)


def test_block_decode_at_validation_errors():
    """The device-position decode validates against max_start_pos on the host."""
    a = dba.ModelArgs(dim=256, n_heads=2, n_kv_heads=1, max_batch_size=2, max_seq_len=16)
    E, U, W = dba._lib.LLAMA_ERR_INVALID_ARG, dba._lib.LLAMA_ERR_UNSUPPORTED, dba._lib.LLAMA_ERR_WORKSPACE_TOO_SMALL
    assert _raw_decode_at(a) == W                            # valid call, workspace missing
    assert _raw_decode_at(a, max_pos=15) == W                # the last cache row
    assert _raw_decode_at(a, max_pos=16) == E                # max_start_pos + 1 > max_seq_len
    assert _raw_decode_at(a, max_pos=-1) == E
    assert _raw_decode_at(a, max_pos=15, freqs_end=15) == E  # RoPE table too short for the largest position
    assert _raw_decode_at(a, pos=None) == E
    assert _raw_decode_at(a, pos=(1 << 22) + 2) == E         # misaligned position pointer
    assert _raw_decode_at(a, bsz=3) == E
    assert _raw_decode_at(a, dtype=dba.LLAMA_F32) == U       # bf16 only
    # the workspace for the largest position suffices
    need = dba.llama_block_workspace_size(a, 1, 1, 15, dba.LLAMA_BF16)
    assert _raw_decode_at(a, max_pos=15, ws_bytes=need - 1) == W


def test_runner_rejects_weights_of_another_shape():
    """The C ABI derives every extent from the model arguments (the FFN width from
    dim, multiple_of and ffn_dim_multiplier); the Python runner checks the weight
    shapes against them before anything reaches the device."""
    from decoder_block_amd.runner import check_weight_shapes, model_args_for
    w = wl.Workload(31, "ffn-width-mismatch", "bf16", 2048, 16, 8, 1024, 256, None, 1e-5, 5e5, batch=1,
                    prefill_len=4, decode_steps=0)
    with pytest.raises(ValueError, match="w1"):
        check_weight_shapes(model_args_for(w), wl.block_weights(w))
    ok = w.scaled(ffn_hidden=1536, ffn_dim_multiplier=0.25)
    check_weight_shapes(model_args_for(ok), wl.block_weights(ok))


def test_every_device_pointer_must_be_aligned():
    """Every tensor pointer an entry point passes to a kernel must be 16-byte aligned
    (int32 id/position arrays and per-row uniforms 4-byte): one pointer at a time is
    moved to an 8-byte (or 2-byte) boundary and the call must return INVALID_ARG.
    Calls with a workspace pass one that is too small, so that a missing alignment
    check would surface as WORKSPACE_TOO_SMALL; no call here reaches a launch."""
    lib = dba.lib()
    E, W = dba._lib.LLAMA_ERR_INVALID_ARG, dba._lib.LLAMA_ERR_WORKSPACE_TOO_SMALL
    BF = dba.LLAMA_BF16
    p = 1 << 20
    m, m4 = p + 8, p + 2

    def each(n, call, bad=m):
        for i in range(n):
            ptrs = [p] * n
            ptrs[i] = bad
            assert call(ptrs) == E, (call, i)

    each(3, lambda q: lib.llama_rmsnorm(*q, 4, 256, 1e-5, BF, None))
    each(3, lambda q: lib.llama_rope(*q, 64, 1, 9, 0, 4, 4, 64, BF, None))
    each(3, lambda q: lib.llama_linear(*q, 4, 128, 64, BF, None))
    a = dba.ModelArgs(dim=512, n_heads=4, n_kv_heads=2, max_batch_size=2, max_seq_len=8)
    c = ctypes.byref(a.c())
    each(6, lambda q: lib.llama_gqa_attn_prefill(*q, c, 1, 4, 0, BF, None))
    big = dba.ModelArgs(dim=8192, n_heads=64, n_kv_heads=8, max_batch_size=1, max_seq_len=9000)
    cb = ctypes.byref(big.c())
    assert lib.llama_gqa_attn_decode(p, p, p, p, p, p, cb, 1, 8000, p, 16, BF, None) == W
    each(7, lambda q: lib.llama_gqa_attn_decode(*q[:6], cb, 1, 8000, q[6], 16, BF, None))
    assert lib.llama_swiglu_ffn(p, p, p, p, p, 4, 256, 768, p, 0, BF, None) == W
    each(6, lambda q: lib.llama_swiglu_ffn(*q[:5], 4, 256, 768, q[5], 0, BF, None))
    # the block: activations, caches, table, workspace and each of the nine weights
    ba = dba.ModelArgs(dim=256, n_heads=2, n_kv_heads=1, max_batch_size=2, max_seq_len=16)
    assert _raw_block_forward(ba) == W
    for name in ("x", "ck", "cv", "freqs", "ws"):
        assert _raw_block_forward(ba, **{name: m}) == E, name
    assert _raw_block_forward(ba, out=2 * p + 8) == E
    for i in range(9):
        ptrs = [p] * 9
        ptrs[i] = m
        assert _raw_block_forward(ba, weights=L.CBlockWeights(*ptrs)) == E, i
    assert _raw_decode_at(ba, ck=m) == E
    # embedding: ids 4-byte, table and output 16-byte
    assert lib.llama_embedding(m4, p, p, 4, 256, 10, BF, None) == E
    each(2, lambda q: lib.llama_embedding(p, *q, 4, 256, 10, BF, None))
    # output projection: h, norm weight, W_out, logits, workspace 16-byte; ids 4-byte
    assert lib.llama_lm_head_argmax(p, 256, p, p, p, p, 2, 256, 1000, 1e-5, p, 0, BF, None) == W
    each(4, lambda q: lib.llama_lm_head_argmax(q[0], 256, q[1], q[2], q[3], p, 2, 256, 1000, 1e-5, p, 0, BF, None))
    assert lib.llama_lm_head_argmax(p, 256, p, p, p, p, 2, 256, 1000, 1e-5, m, 0, BF, None) == E
    assert lib.llama_lm_head_argmax(p, 256, p, p, p, m4, 2, 256, 1000, 1e-5, p, 0, BF, None) == E
    # sampling: logits 16-byte, ids and uniforms 4-byte
    assert lib.llama_sample_top_p(m, p, 4, 100, 0.8, 0.9, p, None) == E
    assert lib.llama_sample_top_p(p, m4, 4, 100, 0.8, 0.9, p, None) == E
    assert lib.llama_sample_top_p(p, p, 4, 100, 0.8, 0.9, m4, None) == E


def test_binding_checks_tensor_extents_before_the_call():
    """Callers that pass tensors straight to the binding (not through BlockRunner) get
    the same host-side extent checks: weights against the shapes the model arguments
    imply, the caches and the activations against the call's extents."""
    import torch
    from decoder_block_amd.runner import model_args_for
    w = wl.Workload(41, "extents", "bf16", 256, 2, 1, 768, 256, None, 1e-5, 1e4, batch=2, prefill_len=4,
                    decode_steps=0)
    a = model_args_for(w)
    wts = wl.block_weights(w)
    shape = (w.batch, w.max_seq_len, w.n_kv_heads, w.head_dim)
    ck, cv = torch.zeros(shape, dtype=torch.bfloat16), torch.zeros(shape, dtype=torch.bfloat16)
    x = torch.zeros(w.batch, 4, w.dim, dtype=torch.bfloat16)
    out = torch.empty_like(x)
    bad = dict(wts, w2=wts["w2"][:, :512].contiguous())
    with pytest.raises(ValueError, match="w2"):
        dba.llama_block_forward(a, bad, ck, cv, 1 << 20, 16, x, out, 2, 4, 0, 1 << 20, 0)
    with pytest.raises(ValueError, match="cache_k"):
        dba.llama_block_forward(a, wts, ck[:1], cv, 1 << 20, 16, x, out, 2, 4, 0, 1 << 20, 0)
    with pytest.raises(ValueError, match="out"):
        dba.llama_block_forward(a, wts, ck, cv, 1 << 20, 16, x, out[:1], 2, 4, 0, 1 << 20, 0)
    with pytest.raises(ValueError, match="x"):
        dba.llama_block_decode_at(a, wts, ck, cv, 1 << 20, 16, x[:, :1][:1], out, 2, 1 << 20, 3, 1 << 20, 0)


def test_static_scratch_decode_refuses_oversized_calls_on_the_host():
    """llama_gqa_attn_decode_static keeps its split-K partials in an 8 MiB static
    array: a call whose partials need more (one sequence, 16 query heads on one kv
    head, 4.2 million attended keys: 8.08 MiB) is refused before anything reaches
    the device; the size check precedes the scratch lookup and every launch."""
    lib = dba.lib()
    assert lib.llama_static_scratch_bytes() == 8 << 20
    a = dba.ModelArgs(dim=2048, n_heads=16, n_kv_heads=1, multiple_of=256, max_batch_size=1, max_seq_len=4_200_001)
    assert dba.llama_attn_decode_workspace_size(a, 1, 4_200_000) > lib.llama_static_scratch_bytes()
    p = 1 << 20
    assert lib.llama_gqa_attn_decode_static(p, p, p, p, p, p, ctypes.byref(a.c()), 1, 4_200_000, dba.LLAMA_BF16,
                                            None) == dba._lib.LLAMA_ERR_SCRATCH_TOO_SMALL
    # argument errors come back as for the workspace call
    assert lib.llama_gqa_attn_decode_static(p, p, p, p, p, p, ctypes.byref(a.c()), 2, 10, dba.LLAMA_BF16,
                                            None) == dba._lib.LLAMA_ERR_INVALID_ARG
    assert "scratch" in dba.status_str(dba._lib.LLAMA_ERR_SCRATCH_TOO_SMALL)
