"""Parity of each C entry point against the CPU oracle on seeded inputs (GPU).

Shapes span several tiles and ragged tails; every call goes through the C ABI
(via the ctypes binding) and every expected value comes from ``oracle``.
"""
import math

import numpy as np
import pytest
import torch

import decoder_block_amd as dba
import workloads as wl
from oracle import block as ob
from tests.gpu_util import check, f64, need_gpu

pytestmark = pytest.mark.gpu

_tid = [100]


def rnd(shape, std=1.0, dtype="bf16"):
    _tid[0] += 1
    return wl.normal(tuple(shape), std, dtype, 0, 0, _tid[0])


def dev(t):
    return t.to("cuda:0")


def tdt(dtype):
    return wl.torch_dtype(dtype)


# ----------------------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,dim", [(37, 256), (129, 4096), (5, 8192), (3, 20480)])
def test_rmsnorm(dtype, rows, dim):
    need_gpu()
    print(f"case rmsnorm {dtype} rows={rows} dim={dim}", flush=True)
    x = rnd((rows, dim), 1.0, dtype) * 3
    w = (1.0 + rnd((dim,), 0.2, dtype)).to(tdt(dtype))
    x = x.to(tdt(dtype))
    y = torch.empty_like(x, device="cuda:0")
    dba.llama_rmsnorm(dev(x), dev(w), y, rows, dim, 1e-5)
    torch.cuda.synchronize()
    ref = ob.rms_norm(f64(x), f64(w), 1e-5)
    check(y, ref, dtype, f"rmsnorm {dtype} {rows}x{dim}")


# ----------------------------------------------------------------------------- RoPE
@pytest.mark.parametrize("head_dim,end,theta", [(128, 16640, 5e5), (64, 4096, 1e4), (32, 200, 1e4)])
def test_rope_table(head_dim, end, theta):
    need_gpu()
    print(f"case rope_freqs d={head_dim} end={end} theta={theta}", flush=True)
    f = torch.empty(end, head_dim // 2, 2, device="cuda:0")
    dba.llama_rope_freqs(f, head_dim, end, theta)
    torch.cuda.synchronize()
    ang = ob.rope_angles(head_dim, range(end), theta)
    got = f64(f)
    # fp64 evaluation rounded once to fp32: within half an fp32 ulp of 1
    assert np.max(np.abs(got[..., 0] - np.cos(ang))) < 1e-7
    assert np.max(np.abs(got[..., 1] - np.sin(ang))) < 1e-7


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_apply(dtype):
    need_gpu()
    B, S, H, Hkv, d, p0 = 2, 37, 8, 2, 128, 11
    print(f"case rope {dtype}", flush=True)
    end = 2 * (p0 + S)
    f = torch.empty(end, d // 2, 2, device="cuda:0")
    dba.llama_rope_freqs(f, d, end, 5e5)
    xq = rnd((B, S, H, d), 1.0, dtype)
    xk = rnd((B, S, Hkv, d), 1.0, dtype)
    gq, gk = dev(xq), dev(xk)
    dba.llama_rope(gq, gk, f, end, B, S, p0, H, Hkv, d)
    torch.cuda.synchronize()
    pos = list(range(p0, p0 + S))
    check(gq, ob.apply_rope(f64(xq), pos, 5e5), dtype, "rope q")
    check(gk, ob.apply_rope(f64(xk), pos, 5e5), dtype, "rope k")


# ----------------------------------------------------------------------------- GEMM
@pytest.mark.parametrize("dtype,M,K,N", [
    ("bf16", 5, 256, 100),        # skinny path, ragged N
    ("bf16", 3, 32, 72),          # small M, K below one 64-wide k-tile
    ("bf16", 17, 96, 300),        # small M, K = 64 + 32 (not whole 64-wide k-tiles)
    ("bf16", 33, 4096, 640),      # small M, LDS-DMA kernel over 64 k-tiles
    ("bf16", 50, 520, 388),       # 64-row path, K tail (520 = 8*64 + 8)
    ("bf16", 300, 1024, 1000),    # large tiles with ragged M and N (LDS-DMA pipeline)
    ("bf16", 200, 1000, 260),     # large tiles, K not a multiple of 32 (register-staged kernel)
    ("bf16", 257, 64, 256),       # a single k-tile pair, one row past a tile
    ("bf16", 1024, 4096, 1536),   # several full 256x256 tiles
    ("bf16", 512, 256, 1024),     # interior tiles only: 16-byte output stores
    ("bf16", 512, 256, 516),      # rows of 516 columns are not 16-byte aligned: 8-byte stores everywhere
    ("bf16", 8192, 128, 4096),    # 512 tiles: each workgroup of the resident grid walks two
    ("bf16", 8200, 192, 4100),    # 561 tiles, ragged M and N, an odd number of k-tiles per tile
    ("bf16", 1, 4096, 6144),      # one token: weight-streaming kernel, whole 512-wide chunks
    ("bf16", 2, 1000, 260),       # K = 512 + 488: the last chunk is ragged
    ("bf16", 4, 14336, 512),      # four tokens, 28 chunks (two in flight per wave, one left over)
    ("bf16", 3, 40, 100),         # K below one chunk: most lanes idle
    ("bf16", 4, 8, 4),            # one lane of one wave holds all of K; a single workgroup
    # 70B-shaped batch-32 decode, one GPU's share under 8-way tensor parallelism: QKV (one kv head,
    # its 8 query heads: 1280 columns) and wo (1024 input features)
    ("bf16", 32, 8192, 1280), ("bf16", 32, 1024, 8192),
    ("f32", 70, 260, 132),
    ("f32", 1, 260, 132),         # fp32 weight stream: K = 256 + 4 (a ragged 256-element chunk)
    ("f32", 4, 1024, 64),         # four tokens, four chunks of 256
])
def test_linear(dtype, M, K, N):
    need_gpu()
    _linear_case(dtype, M, K, N)


def test_linear_seeded_shapes():
    """Twenty-four projection shapes from a seeded generator: 1-4 rows (weight
    streams), 5-64 (small-M tiles, split over K when the grid is short) and
    65-400 rows (large tiles), K a multiple of 8 up to 3072, N of 4 up to 1200."""
    need_gpu()
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(4243)))
    for i in range(24):
        M = int(g.integers(1, 5) if i % 3 == 0 else (g.integers(5, 65) if i % 3 == 1 else g.integers(65, 401)))
        K = 8 * int(g.integers(1, 385))
        N = 4 * int(g.integers(1, 301))
        _linear_case("bf16", M, K, N)


def _linear_case(dtype, M, K, N):
    print(f"case linear {dtype} M={M} K={K} N={N}", flush=True)
    x = rnd((M, K), 1.0, dtype)
    w = rnd((N, K), 0.05, dtype)
    y = torch.empty(M, N, dtype=tdt(dtype), device="cuda:0")
    dba.llama_linear(dev(x), dev(w), y, M, K, N)
    torch.cuda.synchronize()
    check(y, ob.linear(f64(x), f64(w)), dtype, f"linear {M}x{K}x{N}")


@pytest.mark.parametrize("dtype,rows,dim,hidden", [
    ("bf16", 300, 256, 768), ("bf16", 20, 512, 1536), ("bf16", 64, 256, 776), ("f32", 40, 256, 768),
    # small M with split K: w1/w3 in 4 splits; w2 (K = 2816 = 44 k-tiles) in 11 splits of 4
    ("bf16", 9, 1024, 2816),
    # small M, dim = 352 is not whole 64-wide k-tiles (register-staged kernel for w1/w3)
    ("bf16", 7, 352, 1024),
    # one to four tokens: weight-streaming kernels (dim = 512 is one chunk: three waves idle;
    # 640 = 512 + 128 and 1712 = 3 * 512 + 176 end in ragged chunks)
    ("bf16", 1, 512, 1536), ("bf16", 4, 640, 1712), ("bf16", 2, 4096, 14336),
    # fp32 weight streams
    ("f32", 1, 256, 768), ("f32", 3, 260, 772),
    # 70B-shaped batch-32 decode, one GPU's share of the FFN under 8-way tensor parallelism
    ("bf16", 32, 8192, 3584)])
def test_swiglu_ffn(dtype, rows, dim, hidden):
    need_gpu()
    _swiglu_case(dtype, rows, dim, hidden)


def test_swiglu_ffn_seeded_shapes():
    """Twelve FFN shapes from a seeded generator: 1-4, 5-64 and 65-200 rows, dim
    and hidden multiples of 8 (64-1600 and 128-3200)."""
    need_gpu()
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(4244)))
    for i in range(12):
        rows = int(g.integers(1, 5) if i % 3 == 0 else (g.integers(5, 65) if i % 3 == 1 else g.integers(65, 201)))
        dim = 8 * int(g.integers(8, 201))
        hidden = 8 * int(g.integers(16, 401))
        _swiglu_case("bf16", rows, dim, hidden)


def _swiglu_case(dtype, rows, dim, hidden):
    print(f"case swiglu {dtype} rows={rows} dim={dim} hidden={hidden}", flush=True)
    x = rnd((rows, dim), 1.0, dtype)
    w1, w3 = rnd((hidden, dim), 0.05, dtype), rnd((hidden, dim), 0.05, dtype)
    w2 = rnd((dim, hidden), 0.05, dtype)
    y = torch.empty(rows, dim, dtype=tdt(dtype), device="cuda:0")
    nbytes = dba.llama_ffn_workspace_size(rows, dim, hidden, dba.LLAMA_BF16 if dtype == "bf16" else dba.LLAMA_F32)
    ws = torch.full((max(nbytes, 1),), 0xA5, dtype=torch.uint8, device="cuda:0")   # junk on entry
    ref = ob.swiglu_ffn(f64(x), f64(w1), f64(w3), f64(w2))
    # twice on one workspace: the split reductions must leave their counters reusable
    for rep in range(2):
        y.fill_(float("nan"))
        dba.llama_swiglu_ffn(dev(x), dev(w1), dev(w3), dev(w2), y, rows, dim, hidden, ws, nbytes)
        torch.cuda.synchronize()
        check(y, ref, dtype, f"swiglu call {rep}")


# ----------------------------------------------------------------------------- attention
def _args(H, Hkv, d, maxB, maxS, dtype_dim_mult=1):
    return dba.ModelArgs(dim=H * d, n_heads=H, n_kv_heads=Hkv, multiple_of=256, max_batch_size=maxB,
                         max_seq_len=maxS)


@pytest.mark.parametrize("dtype,B,S,p0,H,Hkv,d", [
    ("bf16", 2, 77, 0, 8, 8, 128),      # MHA, ragged query block
    ("bf16", 1, 300, 0, 8, 2, 128),     # GQA n_rep 4
    ("bf16", 2, 130, 50, 16, 2, 128),   # GQA n_rep 8, chunked prefill (start_pos > 0)
    ("bf16", 1, 200, 0, 4, 1, 64),      # MQA, head_dim 64
    ("bf16", 1, 64, 0, 32, 2, 64),      # n_rep 16 (two head groups per kv head)
    ("f32", 1, 40, 9, 8, 2, 32),
])
def test_attn_prefill(dtype, B, S, p0, H, Hkv, d):
    need_gpu()
    _attn_prefill_case(dtype, B, S, p0, H, Hkv, d)


def _spike(cache_rows, positions, factor):
    """Scale whole key rows (all kv heads) at the given positions: scores against them
    jump by that factor, so the running maximum moves in the middle of a row."""
    for t in positions:
        cache_rows[:, t] = (cache_rows[:, t].float() * factor).to(cache_rows.dtype)


def _attn_prefill_case(dtype, B, S, p0, H, Hkv, d, qstd=1.0, spikes=(), factor=1.0):
    print(f"case attn_prefill {dtype} B={B} S={S} p0={p0} H={H} Hkv={Hkv} d={d} q std {qstd} "
          f"key spikes {list(spikes)} x{factor}", flush=True)
    maxS = p0 + S + 3
    args = _args(H, Hkv, d, B + 1, maxS)
    q = rnd((B, S, H, d), qstd, dtype)
    k = rnd((B, S, Hkv, d), 1.0, dtype)
    v = rnd((B, S, Hkv, d), 1.0, dtype)
    ck = torch.zeros(B + 1, maxS, Hkv, d, dtype=tdt(dtype))
    cv = torch.zeros_like(ck)
    if p0:
        ck[:, :p0] = rnd((B + 1, p0, Hkv, d), 1.0, dtype)
        cv[:, :p0] = rnd((B + 1, p0, Hkv, d), 1.0, dtype)
    _spike(ck, [t for t in spikes if t < p0], factor)
    _spike(k, [t - p0 for t in spikes if p0 <= t < p0 + S], factor)
    gck, gcv = dev(ck), dev(cv)
    out = torch.empty(B, S, H * d, dtype=tdt(dtype), device="cuda:0")
    dba.llama_gqa_attn_prefill(dev(q), dev(k), dev(v), gck, gcv, out, args, B, S, p0)
    torch.cuda.synchronize()
    rck, rcv = f64(ck), f64(cv)
    rck[:B, p0:p0 + S] = f64(k)
    rcv[:B, p0:p0 + S] = f64(v)
    np.testing.assert_array_equal(f64(gck), rck)   # append is a copy: bit-exact
    np.testing.assert_array_equal(f64(gcv), rcv)
    ref = ob.gqa_attention(f64(q), rck, rcv, p0)
    check(out, ref, dtype, "attn prefill")


@pytest.mark.parametrize("B,S,p0,H,Hkv,d,qstd,spikes,factor", [
    (2, 300, 0, 8, 2, 128, 10.0, (), 1.0),                   # scores spread over tens of units
    (2, 300, 0, 8, 2, 128, 1.0, (3, 140, 141, 290), 30.0),  # single keys far above the rest, mid-row
    (1, 200, 100, 4, 1, 64, 8.0, (20, 150, 299), 20.0),     # cached and new spikes, MQA, head_dim 64
    (2, 130, 0, 8, 8, 128, 16.0, (64, 65), 8.0),            # MHA, spikes at a tile boundary
])
def test_attn_prefill_sharp_softmax(B, S, p0, H, Hkv, d, qstd, spikes, factor):
    """Sharp score distributions (the pages take the softmax in fp32 after the -inf
    mask): the kernel keeps its running maximum until some row's maximum grows by
    more than 8 in log2 units, so these cases move it in the middle of rows, from
    key tiles of one block to the next, against the oracle's exact softmax."""
    need_gpu()
    _attn_prefill_case("bf16", B, S, p0, H, Hkv, d, qstd, spikes, factor)


def test_attn_prefill_sequences_in_cache_sized_groups():
    """Three 8200-token sequences of GQA 32/16 attend 67 MB of K/V each: more
    than the prefill kernel takes in one dispatch group (192 MiB), so it runs
    the sequences as a group of two, then a group of one.  Sampled query rows
    (first and last of several 64-position query blocks) against the oracle."""
    need_gpu()
    B, S, H, Hkv, d = 3, 8200, 32, 16, 128
    print(f"case attn_prefill grouped B={B} S={S} H={H} Hkv={Hkv} d={d}", flush=True)
    args = _args(H, Hkv, d, B + 1, S + 3)
    q = rnd((B, S, H, d), 1.0)
    k = rnd((B, S, Hkv, d), 1.0)
    v = rnd((B, S, Hkv, d), 1.0)
    gck = torch.zeros(B + 1, S + 3, Hkv, d, dtype=torch.bfloat16, device="cuda:0")
    gcv = torch.zeros_like(gck)
    out = torch.empty(B, S, H * d, dtype=torch.bfloat16, device="cuda:0")
    dba.llama_gqa_attn_prefill(dev(q), dev(k), dev(v), gck, gcv, out, args, B, S, 0)
    torch.cuda.synchronize()
    assert torch.equal(gck[:B, :S].cpu(), k) and torch.equal(gcv[:B, :S].cpu(), v)   # the append: a copy
    rows = [0, 1, 63, 64, 2047, 4100, 8135, 8199]
    ref = ob.gqa_attention(f64(q), f64(k), f64(v), 0, rows)
    check(out[:, rows], ref, "bf16", "attn prefill, sequences in groups")


@pytest.mark.parametrize("dtype,B,p0,H,Hkv,d", [
    ("bf16", 3, 0, 8, 2, 128),       # single key
    ("bf16", 2, 40, 8, 8, 128),      # MHA, short
    ("bf16", 4, 4096, 64, 8, 128),   # 70B-shaped group, long context
    ("bf16", 1, 8300, 32, 8, 128),   # many splits
    ("bf16", 2, 999, 4, 1, 64),      # MQA head_dim 64
    ("bf16", 1, 500, 32, 1, 128),    # n_rep 32 (two head groups)
    ("bf16", 2, 300, 8, 2, 64),      # three splits, head_dim 64 (one-wave merge)
    ("bf16", 16, 1500, 16, 8, 128),  # 128 (sequence, kv head) units: one 8-wave workgroup each, no split
    ("bf16", 64, 700, 8, 4, 64),     # 256 units, head_dim 64, 8 waves
    ("bf16", 32, 4096, 8, 1, 128),   # 70B shape at batch 32, one GPU's share under 8-way TP: 1 kv head, n_rep 8
    ("f32", 2, 79, 8, 2, 32),
])
def test_attn_decode(dtype, B, p0, H, Hkv, d):
    need_gpu()
    _attn_decode_case(dtype, B, p0, H, Hkv, d)


def test_attn_decode_seeded_shapes():
    """Twenty decode shapes drawn from a seeded generator (batch 1-64, 0-3000
    cached keys, 1-8 kv heads, n_rep 1-32, head_dim 64/128): they land on every
    grid rule of the decode kernel (one split, merged by one wave per row or by
    four, one 8-wave workgroup per unit)."""
    need_gpu()
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(4242)))
    for _ in range(20):
        Hkv = int(g.choice([1, 2, 4, 8]))
        n_rep = int(g.choice([1, 2, 4, 8, 16, 32]))
        while Hkv * n_rep > 64:
            n_rep //= 2
        d = int(g.choice([64, 128]))
        B = int(g.integers(1, 65))
        # keep the oracle's expanded float64 cache under ~400 MB
        p0_max = max(1, min(3000, int(5e7 // (B * Hkv * n_rep * d))))
        p0 = int(g.integers(0, p0_max + 1))
        _attn_decode_case("bf16", B, p0, Hkv * n_rep, Hkv, d)


def _attn_decode_case(dtype, B, p0, H, Hkv, d, qstd=1.0, spikes=(), factor=1.0):
    print(f"case attn_decode {dtype} B={B} p0={p0} H={H} Hkv={Hkv} d={d} q std {qstd} "
          f"key spikes {list(spikes)} x{factor}", flush=True)
    maxS = p0 + 2
    args = _args(H, Hkv, d, B, maxS)
    q = rnd((B, 1, H, d), qstd, dtype)
    k = rnd((B, 1, Hkv, d), 1.0, dtype)
    v = rnd((B, 1, Hkv, d), 1.0, dtype)
    ck = torch.zeros(B, maxS, Hkv, d, dtype=tdt(dtype))
    cv = torch.zeros_like(ck)
    if p0:
        ck[:, :p0] = rnd((B, p0, Hkv, d), 1.0, dtype)
        cv[:, :p0] = rnd((B, p0, Hkv, d), 1.0, dtype)
    _spike(ck, [t for t in spikes if t < p0], factor)
    if p0 in spikes:
        k = (k.float() * factor).to(k.dtype)
    gck, gcv = dev(ck), dev(cv)
    out = torch.empty(B, 1, H * d, dtype=tdt(dtype), device="cuda:0")
    nbytes = dba.llama_attn_decode_workspace_size(args, B, p0)
    # a workspace full of junk: the split partials overwrite it, nothing may read it first
    ws = torch.full((max(nbytes, 1),), 0xA5, dtype=torch.uint8, device="cuda:0")
    dba.llama_gqa_attn_decode(dev(q), dev(k), dev(v), gck, gcv, out, args, B, p0, ws, nbytes)
    torch.cuda.synchronize()
    rck, rcv = f64(ck), f64(cv)
    rck[:, p0] = f64(k)[:, 0]
    rcv[:, p0] = f64(v)[:, 0]
    np.testing.assert_array_equal(f64(gck), rck)
    ref = ob.gqa_attention(f64(q), rck, rcv, p0)
    check(out, ref, dtype, "attn decode")


@pytest.mark.parametrize("B,p0,H,Hkv,d,qstd,spikes,factor", [
    (1, 8300, 32, 8, 128, 1.0, (5, 2000, 4100, 8250, 8300), 30.0),   # dozens of splits, four-wave merge
    (1, 8300, 32, 8, 128, 12.0, (), 1.0),                            # every split sharp
    (4, 1500, 8, 2, 128, 1.0, (7, 700, 1499), 25.0),                 # about a dozen splits, one-wave merge
    (2, 300, 8, 2, 64, 10.0, (150, 300), 20.0),                      # three splits, head_dim 64
    (16, 1500, 16, 8, 128, 1.0, (100, 900, 1400), 30.0),             # one 8-wave workgroup per unit, no split
])
def test_attn_decode_sharp_softmax(B, p0, H, Hkv, d, qstd, spikes, factor):
    """Sharp score distributions in decode: single keys far above the rest (in
    different splits, so the split maxima differ by tens of units and the
    log-sum-exp merge weighs most splits by tiny factors) and queries of large
    norm, against the oracle's exact softmax, for the split layouts of the
    decode kernel and both merge kernels."""
    need_gpu()
    _attn_decode_case("bf16", B, p0, H, Hkv, d, qstd, spikes, factor)


# ----------------------------------------------------------------------------- config-5 pieces
@pytest.mark.parametrize("B", [6, 2])   # 2 rows: the weight-streaming kernel computes the logits
def test_embedding_and_lm_head_argmax(B):
    need_gpu()
    print(f"case embedding + lm_head B={B}", flush=True)
    V, D = 1000, 256
    table = rnd((V, D), 0.02)
    tok = torch.tensor([0, 999, 5, 17, 5, 300][:B], dtype=torch.int32)
    out = torch.empty(B, D, dtype=torch.bfloat16, device="cuda:0")
    dba.llama_embedding(dev(tok), dev(table), out, B, D, V)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(out), f64(table)[tok.numpy()])
    h = rnd((B, 3, D), 1.0)             # take the last of 3 rows per sequence (row stride 3*D)
    w_out = rnd((V, D), 0.05)
    # an exact tie: ids 77 and 100 give equal logits.  Both lie in one 128-column
    # tile of the small-M projection, whose k-tiles are summed in a tile-dependent
    # (rotated) order: equal rows in different tiles agree only to rounding.
    w_out[77] = w_out[100]
    norm_w = (1.0 + rnd((D,), 0.2)).to(torch.bfloat16)      # a non-unit final-norm weight
    logits = torch.empty(B, V, dtype=torch.float32, device="cuda:0")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda:0")
    nbytes = dba.llama_lm_head_workspace_size(B, D, V, dba.LLAMA_BF16)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda:0")
    gh = dev(h)
    dba.llama_lm_head_argmax(gh[:, 2], 3 * D, dev(norm_w), dev(w_out), logits, nxt, B, D, V, 1e-5, ws, nbytes)
    torch.cuda.synchronize()
    ref = ob.linear(ob.rms_norm(f64(h)[:, 2], f64(norm_w), 1e-5), f64(w_out))
    e = check(logits, ref, "bf16", "lm head logits")
    got = nxt.cpu().numpy()
    lg = f64(logits)
    assert np.all(lg[:, 77] == lg[:, 100])
    for b in range(B):
        # the argmax of the GPU's own logits, lowest id on ties (exact, integer)
        assert got[b] == int(np.argmax(lg[b]))
        # and a correct greedy token against the exact logits (margin rule)
        assert ref[b, got[b]] >= ref[b].max() - 2 * e["raw_maxabs"]
