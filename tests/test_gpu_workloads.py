"""Whole-block parity at the workloads' real shapes and GPU-side invariants (GPU).

The block runs through ``llama_block_forward``; the oracle evaluates the same
seeded inputs.  At full size the oracle evaluates sampled output rows (each
output row has its own definition) and the whole KV cache.  A decode step at
position p equals the prefill row at p (pinned on the oracle by
test_kv_cache_decode_equals_full_prefill), so decode rows are checked against
the oracle's rows of one call over all positions.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from decoder_block_amd.runner import BlockRunner, model_args_for
from oracle import block as ob
from tests.gpu_util import check, f64, need_gpu

pytestmark = pytest.mark.gpu


# RMSNorm weights 1 + N(0, 0.2^2), distinct per norm and layer: the five workloads
# use unit weights, so these tests exercise the gain multiply of each fused
# normalisation (row-scale form, one-to-four-token weight streams, the split
# reduction of 5-64 tokens) and the bf16 rounding of x * g
GAINS = "normal"


def _w64(wts):
    return {k: v.to(torch.float64).numpy() for k, v in wts.items()}


def _rows(S, extra=()):
    r = {0, 1, 2, 63, 64, 127, 128, 255, 256, S // 2, S - 2, S - 1, *extra}
    return sorted(x for x in r if 0 <= x < S)


def test_tiny_f32_prefill_then_decode_steps():
    dev = need_gpu()
    w = wl.WORKLOADS[1]
    print(f"case {w.name}: prefill {w.prefill_len} + {w.decode_steps} decode steps (f32)", flush=True)
    wts = wl.block_weights(w)
    x = wl.activations(w)
    run = BlockRunner(model_args_for(w), wts, torch.float32, dev)
    S = w.prefill_len
    outs = [run.forward(x[:, :S].contiguous().to(dev), 0)]
    for t in range(w.decode_steps):
        outs.append(run.forward(x[:, S + t:S + t + 1].contiguous().to(dev), S + t))
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=1)
    W = _w64(wts)
    shape = (w.batch, w.max_seq_len, w.n_kv_heads, w.head_dim)
    ck, cv = np.zeros(shape), np.zeros(shape)
    xr = f64(x)
    ref = [ob.block_forward(xr[:, :S], W, ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)]
    for t in range(w.decode_steps):
        ref.append(ob.block_forward(xr[:, S + t:S + t + 1], W, ck, cv, S + t, w.n_heads, w.n_kv_heads, w.norm_eps,
                                    w.rope_theta))
    check(got, np.concatenate(ref, axis=1), "f32", "tiny block outputs")
    check(run.cache_k, ck, "f32", "tiny cache_k")
    check(run.cache_v, cv, "f32", "tiny cache_v")


def test_llama7b_block_prefill_full_size():
    dev = need_gpu()
    w = wl.WORKLOADS[2]
    print(f"case {w.name}: B={w.batch} S={w.prefill_len} bf16", flush=True)
    wts = wl.block_weights(w)
    x = wl.activations(w)
    run = BlockRunner(model_args_for(w), wts, torch.bfloat16, dev)
    out = run.forward(x.to(dev), 0)
    torch.cuda.synchronize()
    rows = _rows(w.prefill_len)
    shape = (w.batch, w.max_seq_len, w.n_kv_heads, w.head_dim)
    ck, cv = np.zeros(shape), np.zeros(shape)
    ref = ob.block_forward(f64(x), _w64(wts), ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta,
                           rows=rows)
    check(out[:, rows], ref, "bf16", "7B block sampled rows")
    check(run.cache_k, ck, "bf16", "7B cache_k (k after RoPE)")
    check(run.cache_v, cv, "bf16", "7B cache_v")


def test_llama3_8b_block_prefill_chunked_prefill_and_128_decodes():
    dev = need_gpu()
    w = wl.WORKLOADS[3]
    print(f"case {w.name}: prefill {w.prefill_len} + {w.decode_steps} decodes bf16", flush=True)
    wts = wl.block_weights(w)
    x = wl.activations(w)
    run = BlockRunner(model_args_for(w), wts, torch.bfloat16, dev)
    S = w.prefill_len
    gx = x.to(dev)
    pre = run.forward(gx[:, :S].contiguous(), 0)
    dec = [run.forward(gx[:, S + t:S + t + 1].contiguous(), S + t) for t in range(w.decode_steps)]
    # the same prompt fed as 4 chunks of 2048 tokens (start_pos 0, 2048, 4096, 6144)
    runc = BlockRunner(model_args_for(w), wts, torch.bfloat16, dev)
    C = 2048
    chunked = torch.cat([runc.forward(gx[:, c:c + C].contiguous(), c) for c in range(0, S, C)], dim=1)
    torch.cuda.synchronize()
    got = torch.cat([pre] + dec, dim=1)
    prompt_rows = _rows(S, (2047, 2048, 4095, 4096, 6143, 6144))
    rows = prompt_rows + [S + t for t in (0, 1, 2, 31, 63, 64, 126, 127)]
    shape = (w.batch, w.max_seq_len, w.n_kv_heads, w.head_dim)
    ck, cv = np.zeros(shape), np.zeros(shape)
    ref = ob.block_forward(f64(x), _w64(wts), ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta,
                           rows=rows)
    check(got[:, rows], ref, "bf16", "8B block sampled prefill + decode rows")
    check(run.cache_k, ck, "bf16", "8B cache_k")
    check(run.cache_v, cv, "bf16", "8B cache_v")
    check(chunked[:, prompt_rows], ref[:, :len(prompt_rows)], "bf16", "8B chunked prefill (4 x 2048) sampled rows")
    check(runc.cache_k[:, :S], ck[:, :S], "bf16", "8B chunked prefill cache_k")
    check(runc.cache_v[:, :S], cv[:, :S], "bf16", "8B chunked prefill cache_v")


def test_llama2_70b_block_decode_batch32():
    dev = need_gpu()
    w = wl.WORKLOADS[4]
    print(f"case {w.name}: B={w.batch} decode at {w.cache_prefill} bf16", flush=True)
    wts = wl.block_weights(w)
    x = wl.activations(w)
    ck0, cv0 = wl.prefilled_cache(w)
    run = BlockRunner(model_args_for(w), wts, torch.bfloat16, dev, cache=(ck0, cv0))
    out = run.forward(x.to(dev), w.cache_prefill)
    torch.cuda.synchronize()
    ck, cv = f64(ck0), f64(cv0)
    ref = ob.block_forward(f64(x), _w64(wts), ck, cv, w.cache_prefill, w.n_heads, w.n_kv_heads, w.norm_eps,
                           w.rope_theta)
    check(out, ref, "bf16", "70B decode outputs")
    p = w.cache_prefill
    check(run.cache_k[:, p], ck[:, p], "bf16", "70B appended k")
    check(run.cache_v[:, p], cv[:, p], "bf16", "70B appended v")
    # rows before the append are untouched (bit-exact)
    np.testing.assert_array_equal(f64(run.cache_k[:, :p]), f64(ck0[:, :p]))


def test_block_decode_seeded_shapes():
    """Ten one-token block calls with shapes from a seeded generator (head_dim
    64/128, 1-8 kv heads, n_rep 1-8, batch 1-80 over 1-1500 cached N(0,1) rows,
    non-unit RMSNorm weights):
    weight streams with the norms fused (1-4 tokens), small-M tiles with wo's
    split reduction fused with ffn_norm (5-64), large tiles beyond; outputs and
    the appended cache rows against the oracle."""
    dev = need_gpu()
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(4245)))
    for i in range(10):
        d = int(g.choice([64, 128]))
        Hkv = int(g.choice([1, 2, 4, 8]))
        n_rep = int(g.choice([1, 2, 4, 8]))
        while Hkv * n_rep * d > 4096:
            n_rep //= 2
        H = Hkv * n_rep
        D = H * d
        mo = int(g.choice([8, 64, 256]))
        F = mo * -(-int(8 * D / 3) // mo)
        B = int(g.integers(1, 5) if i % 3 == 0 else (g.integers(5, 65) if i % 3 == 1 else g.integers(65, 81)))
        p0 = int(g.integers(1, 1501))
        w = wl.Workload(200 + i, f"seeded-{i}", "bf16", D, H, Hkv, F, mo, None, 1e-5, 1e4, batch=B, prefill_len=0,
                        decode_steps=1, cache_prefill=p0, norm_gains=GAINS)
        print(f"case {w.name}: D={D} H={H} Hkv={Hkv} d={d} F={F} B={B} decode at {p0}", flush=True)
        wts = wl.block_weights(w)
        x = wl.activations(w)
        ck0, cv0 = wl.prefilled_cache(w)
        run = BlockRunner(model_args_for(w), wts, torch.bfloat16, dev, cache=(ck0, cv0))
        out = run.forward(x.to(dev), p0)
        torch.cuda.synchronize()
        ck, cv = f64(ck0), f64(cv0)
        ref = ob.block_forward(f64(x), _w64(wts), ck, cv, p0, H, Hkv, w.norm_eps, w.rope_theta)
        check(out, ref, "bf16", f"{w.name} decode outputs")
        check(run.cache_k[:, p0], ck[:, p0], "bf16", f"{w.name} appended k")
        check(run.cache_v[:, p0], cv[:, p0], "bf16", f"{w.name} appended v")
        del run
        torch.cuda.empty_cache()


def test_block_prefill_seeded_shapes():
    """Eight block prefill calls with shapes from a seeded generator (head_dim
    64/128, 1-8 kv heads, n_rep 1-8, batch 1-4, 5-700 new tokens after 0-500
    cached N(0,1) rows, non-unit RMSNorm weights): ragged token counts on every GEMM tile family, the
    attention's head grouping and causal offsets; outputs and the appended cache
    rows against the oracle."""
    dev = need_gpu()
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(4246)))
    for i in range(8):
        d = int(g.choice([64, 128]))
        Hkv = int(g.choice([1, 2, 4, 8]))
        n_rep = int(g.choice([1, 2, 4, 8]))
        while Hkv * n_rep * d > 2048:
            n_rep //= 2
        H = Hkv * n_rep
        D = H * d
        mo = int(g.choice([8, 64, 256]))
        F = mo * -(-int(8 * D / 3) // mo)
        B = int(g.integers(1, 5))
        S = int(g.integers(5, 701))
        p0 = int(g.choice([0, int(g.integers(1, 501))]))
        w = wl.Workload(300 + i, f"seeded-prefill-{i}", "bf16", D, H, Hkv, F, mo, None, 1e-5, 1e4, batch=B,
                        prefill_len=S, decode_steps=0, cache_prefill=p0, norm_gains=GAINS)
        print(f"case {w.name}: D={D} H={H} Hkv={Hkv} d={d} F={F} B={B} S={S} at {p0}", flush=True)
        wts = wl.block_weights(w)
        x = wl.activations(w)[:, :S].contiguous()
        ck0, cv0 = wl.prefilled_cache(w)
        run = BlockRunner(model_args_for(w), wts, torch.bfloat16, dev, cache=(ck0, cv0))
        out = run.forward(x.to(dev), p0)
        torch.cuda.synchronize()
        ck, cv = f64(ck0), f64(cv0)
        ref = ob.block_forward(f64(x), _w64(wts), ck, cv, p0, H, Hkv, w.norm_eps, w.rope_theta)
        check(out, ref, "bf16", f"{w.name} outputs")
        check(run.cache_k[:, p0:p0 + S], ck[:, p0:p0 + S], "bf16", f"{w.name} appended k")
        check(run.cache_v[:, p0:p0 + S], cv[:, p0:p0 + S], "bf16", f"{w.name} appended v")
        del run
        torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- invariants
SMALL = wl.Workload(30, "small-gqa", "bf16", 512, 8, 2, 1536, 256, None, 1e-5, 1e4, batch=3, prefill_len=100,
                    decode_steps=6, norm_gains=GAINS)
# 8 kv heads of head_dim 128: decode attention takes its one-workgroup-per-row layout
SMALL_ROWS = wl.Workload(31, "small-gqa-8kv", "bf16", 2048, 16, 8, 1536, 256, 0.25, 1e-5, 5e5, batch=3,
                         prefill_len=100, decode_steps=6, norm_gains=GAINS)


# one to four tokens per decode step run the weight-streaming projections with the
# normalisation fused; dim 640 = 512 + 128 and hidden 1712 = 3 * 512 + 176 end in
# ragged chunks, and a single kv head serves all five query heads
RAGGED4 = wl.Workload(32, "ragged-640-b4", "bf16", 640, 5, 1, 1712, 8, None, 1e-5, 1e4, batch=4, prefill_len=45,
                      decode_steps=4, norm_gains=GAINS)
# six tokens per decode step: the split-K projections of the tiled kernels, with
# wo's split reduction fused with the residual add and ffn_norm
SMALL_ROWS6 = wl.Workload(34, "small-gqa-8kv-b6", "bf16", 2048, 16, 8, 1536, 256, 0.25, 1e-5, 5e5, batch=6,
                          prefill_len=100, decode_steps=4, norm_gains=GAINS)
# 16 sequences x 8 kv heads = 128 units: decode attention runs one 8-wave workgroup per
# unit (no split), also with the position read from device memory
SMALL_ROWS16 = wl.Workload(35, "small-gqa-8kv-b16", "bf16", 2048, 16, 8, 1536, 256, 0.25, 1e-5, 5e5, batch=16,
                           prefill_len=100, decode_steps=4, norm_gains=GAINS)
RAGGED1 = wl.Workload(33, "ragged-640-b1", "bf16", 640, 5, 1, 1712, 8, None, 1e-5, 1e4, batch=1, prefill_len=45,
                      decode_steps=4, norm_gains=GAINS)
# three tokens per decode step over 300-302 cached rows: the weight-streaming
# projections, and decode attention in three splits whose partials live in the
# workspace
SPLIT3 = wl.Workload(37, "small-gqa-8kv-b3-split", "bf16", 2048, 16, 8, 1536, 256, 0.25, 1e-5, 5e5, batch=3,
                     prefill_len=300, decode_steps=3, norm_gains=GAINS)
# 40 tokens per decode step: 64-row tiles over 40 rows (a ragged row tail) with K split
SMALL_ROWS40 = wl.Workload(36, "small-gqa-8kv-b40", "bf16", 2048, 16, 8, 1536, 256, 0.25, 1e-5, 5e5, batch=40,
                           prefill_len=100, decode_steps=3, norm_gains=GAINS)


def _small_runner(dev, batch=None, w=SMALL):
    return BlockRunner(model_args_for(w, max_batch=batch or w.batch), wl.block_weights(w), torch.bfloat16, dev)


@pytest.mark.parametrize("w", [SMALL, SMALL_ROWS, SMALL_ROWS6, RAGGED4, RAGGED1], ids=lambda w: w.name)
def test_decode_chain_matches_prefill_and_oracle(w):
    dev = need_gpu()
    print(f"case {w.name}: prefill + decode chain + chunked prefill", flush=True)
    x = wl.activations(w).to(dev)
    a = w.prefill_len
    full = _small_runner(dev, w=w).forward(x, 0)
    r = _small_runner(dev, w=w)
    parts = [r.forward(x[:, :a].contiguous(), 0)]
    parts += [r.forward(x[:, a + t:a + t + 1].contiguous(), a + t) for t in range(w.decode_steps)]
    chunk = _small_runner(dev, w=w)
    c = [chunk.forward(x[:, :40].contiguous(), 0), chunk.forward(x[:, 40:].contiguous(), 40)]
    torch.cuda.synchronize()
    chain = torch.cat(parts, dim=1)
    chunked = torch.cat(c, dim=1)
    shape = (w.batch, w.max_seq_len, w.n_kv_heads, w.head_dim)
    ck, cv = np.zeros(shape), np.zeros(shape)
    ref = ob.block_forward(f64(x), _w64(wl.block_weights(w)), ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps,
                           w.rope_theta)
    check(full, ref, "bf16", "small prefill")
    check(chain, ref, "bf16", "small prefill + decode chain")
    check(chunked, ref, "bf16", "small chunked prefill")
    check(chain, f64(full), "bf16", "chain vs full prefill (GPU vs GPU)")


@pytest.mark.parametrize("w", [SPLIT3, SMALL_ROWS6, SMALL_ROWS16, SMALL_ROWS40], ids=lambda w: w.name)
def test_decode_step_ignores_workspace_contents(w):
    """1-4 tokens: the attention's split partials live in the workspace; 5-64
    tokens: the projections split K through fp32 partial tiles in the workspace
    (wo's reduction fused with ffn_norm).  Each decode step runs three
    times: over a workspace with every bit set, over a zeroed one, and over the
    previous call's leftovers; the outputs must agree bit for bit and follow the
    oracle's prefill + decode chain (40 rows: 64-row tiles with a ragged tail)."""
    dev = need_gpu()
    print(f"case {w.name}: decode steps over filled, zeroed and reused workspaces", flush=True)
    x = wl.activations(w).to(dev)
    a = w.prefill_len
    r = _small_runner(dev, w=w)
    parts = [r.forward(x[:, :a].contiguous(), 0)]
    for t in range(w.decode_steps):
        xt = x[:, a + t:a + t + 1].contiguous()
        r.reserve(w.batch, 1, a + t)
        r.ws.fill_(255)
        o1 = r.forward(xt, a + t).clone()
        r.ws.zero_()
        o2 = r.forward(xt, a + t).clone()
        o3 = r.forward(xt, a + t).clone()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"step {t}: a workspace with every bit set changed the output"
        assert torch.equal(o2, o3), f"step {t}: the previous call's workspace contents changed the output"
        parts.append(o1)
    chain = torch.cat(parts, dim=1)
    n = a + w.decode_steps
    shape = (w.batch, w.max_seq_len, w.n_kv_heads, w.head_dim)
    ck, cv = np.zeros(shape), np.zeros(shape)
    ref = ob.block_forward(f64(x[:, :n]), _w64(wl.block_weights(w)), ck, cv, 0, w.n_heads, w.n_kv_heads,
                           w.norm_eps, w.rope_theta)
    check(chain, ref, "bf16", "prefill + decode chain")
    check(r.cache_k[:, :n], ck[:, :n], "bf16", "cache_k rows")


def test_determinism_batch_independence_causality():
    dev = need_gpu()
    w = SMALL
    x = wl.activations(w)[:, :w.prefill_len].contiguous().to(dev)
    r = _small_runner(dev)
    o1 = r.forward(x, 0).clone()
    o2 = r.forward(x, 0).clone()
    assert torch.equal(o1, o2), "repeated runs differ"
    one = _small_runner(dev, batch=1).forward(x[1:2].contiguous(), 0)
    assert torch.equal(one, o1[1:2]), "batch rows are not independent"
    t = 57
    xp = x.clone()
    xp[:, t] += 1.0
    o3 = r.forward(xp, 0)
    torch.cuda.synchronize()
    assert torch.equal(o3[:, :t], o1[:, :t]), "an output before the perturbed position changed"
    assert not torch.equal(o3[:, t], o1[:, t])


@pytest.mark.parametrize("max_pos", [4000, 1000, 137])
@pytest.mark.parametrize("w", [SMALL, SMALL_ROWS, SMALL_ROWS16], ids=lambda w: w.name)
def test_decode_at_device_position_matches_oracle(w, max_pos):
    """llama_block_decode_at reads the position from device memory.  With a bound
    above the actual position (max_start_pos 4000, 1000 or 137 while the steps run at
    100..105) the attention splits are laid out for the bound's length, and the
    later ones are empty (bound 1000: eight splits, merged by one wave per
    row); the outputs and the appended cache rows must still follow the
    oracle's prefill + decode chain."""
    from decoder_block_amd import _lib as L
    dev = need_gpu()
    a = w.prefill_len
    print(f"case {w.name}: device-position decode at {a}..{a + w.decode_steps - 1}, bound {max_pos}", flush=True)
    args = model_args_for(w, max_seq=max_pos + 1)
    r = BlockRunner(args, wl.block_weights(w), torch.bfloat16, dev)
    x = wl.activations(w).to(dev)
    parts = [r.forward(x[:, :a].contiguous(), 0)]
    need = L.llama_block_workspace_size(args, w.batch, 1, max_pos, L.LLAMA_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    pos = torch.empty(1, dtype=torch.int32, device=dev)
    for t in range(w.decode_steps):
        pos.fill_(a + t)
        xt = x[:, a + t:a + t + 1].contiguous()
        out = torch.empty_like(xt)
        L.llama_block_decode_at(args, r.cw, r.cache_k, r.cache_v, r.freqs, r.freqs_end, xt, out, w.batch, pos,
                                max_pos, ws, need)
        parts.append(out)
    torch.cuda.synchronize()
    chain = torch.cat(parts, dim=1)
    shape = (w.batch, w.max_seq_len, w.n_kv_heads, w.head_dim)
    ck, cv = np.zeros(shape), np.zeros(shape)
    n = a + w.decode_steps
    ref = ob.block_forward(f64(x[:, :n]), _w64(wl.block_weights(w)), ck, cv, 0, w.n_heads, w.n_kv_heads,
                           w.norm_eps, w.rope_theta)
    check(chain, ref, "bf16", "prefill + device-position decode chain")
    check(r.cache_k[:, :n], ck[:, :n], "bf16", "cache_k rows")
    check(r.cache_v[:, :n], cv[:, :n], "bf16", "cache_v rows")
    assert not torch.any(r.cache_k[:, n:]), "rows past the last position must stay untouched"
