"""Benchmark of the LLaMA decoder-block forward pass on one MI355X.

One step = one prefill call of the 32-layer Llama-3-8B-shaped stack (dim 4096,
32 query / 8 kv heads, FFN 14336, vocab 128256, bf16) over 64 prompts of 2048
random token ids: the embedding gather, 32 x ``llama_block_forward`` (every
step of the block: RMSNorm, QKV + RoPE + cache append, causal GQA attention,
wo + residual, RMSNorm, w1/w3 + SwiGLU, w2 + residual), the final RMSNorm, the
output projection of the last position and the greedy token, on seeded
synthetic inputs already resident in HBM.  ``value`` is prefill tokens/s per
block: 64 x 2048 tokens x 32 blocks / the step's wall time.

The same JSON line reports the stack's greedy decode (256 one-token steps from
the prefilled caches, eager and replayed from one HIP graph, and with
temperature + top-p sampling), per-stage times from HIP events recorded on the
launch stream, the MFMA roofline fraction of the dominant kernel (the dual
w1/w3 GEMM at M = 131072), the single-block workloads (LLaMA-7B-shaped prefill,
Llama-3-8B-shaped prefill and decode, Llama-2-70B-shaped batch-32 decode, the
tiny fp32 block) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "prefill tokens/s per block + decode step µs; % of MFMA / HBM roofline"
STAGES = ["attention_norm", "qkv_rope_append", "attention", "wo_residual", "ffn_norm", "w1w3_swiglu",
          "w2_residual"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stage_work(w, bsz, S, p0):
    """Algorithmic flops (GEMMs, attention) and bytes (norms) per stage for one call."""
    D, H, Hkv, d, F = w.dim, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn_hidden
    N = bsz * S
    causal_keys = sum(p0 + s + 1 for s in range(S)) if S > 1 else (p0 + 1)
    return {
        "attention_norm": ("hbm", 2 * N * D * 2 + 2 * D),
        "qkv_rope_append": ("mfma", 2 * N * D * (H + 2 * Hkv) * d),
        "attention": ("mfma", 4 * bsz * H * d * causal_keys),
        "wo_residual": ("mfma", 2 * N * H * d * D),
        "ffn_norm": ("hbm", 2 * N * D * 2 + 2 * D),
        "w1w3_swiglu": ("mfma", 4 * N * D * F),
        "w2_residual": ("mfma", 2 * N * F * D),
    }


def decode_bytes(w, bsz, T):
    """HBM bytes of one decode step: weights once, KV cache read, activations."""
    D, H, Hkv, d, F = w.dim, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn_hidden
    weights = 2 * (D * (H + 2 * Hkv) * d + H * d * D + 3 * D * F) + 4 * D
    kv = 2 * 2 * bsz * T * Hkv * d
    return weights, kv


def make_runner(wid, dev, cache=None):
    import torch
    import workloads as wl
    from decoder_block_amd.runner import BlockRunner, model_args_for
    w = wl.WORKLOADS[wid]
    wts = wl.block_weights(w)
    r = BlockRunner(model_args_for(w), wts, torch.bfloat16, dev, cache=cache)
    return w, wts, r


def time_prefill(r, x, steps, warmup, p0=0):
    import torch
    bsz, S, _ = x.shape
    r.reserve(bsz, S, p0)
    out = torch.empty_like(x)
    for _ in range(warmup):
        r.forward(x, p0, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.forward(x, p0, out)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # per-stage durations from HIP events recorded on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(steps)]
    for e in evs:
        r.forward(x, p0, out, events=e)
    torch.cuda.synchronize()
    stage_ms = [sum(e[i - 1].elapsed_time(e[i]) for e in evs) / steps for i in range(1, 8)]
    return wall, stage_ms


def time_chunked_prefill(r, x, chunk, steps, warmup):
    """One prompt fed as consecutive chunks (start_pos 0, chunk, 2*chunk, ...): wall time per whole prompt."""
    import torch
    bsz, S, _ = x.shape
    r.reserve(bsz, chunk, S - chunk)
    parts = [x[:, c:c + chunk].contiguous() for c in range(0, S, chunk)]
    outs = [torch.empty_like(p) for p in parts]

    def once():
        for i, (p, o) in enumerate(zip(parts, outs)):
            r.forward(p, i * chunk, o)
    for _ in range(warmup):
        once()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        once()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def flush_mall(buf):
    """Evicts the 256 MB Infinity Cache (and L2) between decode reps by READING 1 GiB.

    A write-based flush leaves dirty lines whose write-back then competes with
    the timed step's weight stream (measured: a cold 896 MiB read drops from
    6.2 to 4.5 TB/s after a 512 MiB memset), which is not what a decode step
    sees after the previous layer's (read-only) weight stream.
    """
    buf.sum()


def pct(v, q):
    """The q-quantile of the samples v (nearest rank)."""
    s = sorted(v)
    return s[min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))]


def time_decode(r, xs, p0s, flush):
    """Times each one-token call separately (MALL flushed before each): the step
    between two events around the call, then the stages in a second pass with an
    event after each stage (each event adds a few microseconds of its own, so
    the stages are not summed into the step time).  Repeating a call at the same
    position rewrites the same cache row with the same values."""
    import torch
    bsz = xs[0].shape[0]
    r.reserve(bsz, 1, max(p0s))
    out = torch.empty_like(xs[0])
    r.forward(xs[0], p0s[0], out)          # untimed: loads the kernels' code on first use
    torch.cuda.synchronize()
    tot, stage_tot = [], [0.0] * 7
    for x, p0 in zip(xs, p0s):
        flush_mall(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        r.forward(x, p0, out)
        e1.record()
        torch.cuda.synchronize()
        tot.append(e0.elapsed_time(e1))
        flush_mall(flush)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
        r.forward(x, p0, out, events=e)
        torch.cuda.synchronize()
        for i in range(1, 8):
            stage_tot[i - 1] += e[i - 1].elapsed_time(e[i])
    n = len(xs)
    return tot, [s / n for s in stage_tot]


def sources_hash(paths):
    """sha256 (16 hex digits) over the kernel's source files, in the given order."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_traffic(kernel_key):
    """HBM traffic per launch from the committed rocprofv3 PMC summary, or None when the
    kernel source changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            d = json.load(f)
        ent = d[kernel_key]
        return ent["bytes_per_launch"] if sources_hash(ent["sources"]) == ent["sources_sha256_16"] else None
    except Exception:
        return None


def blas_threads():
    """(threads, library) of the BLAS numpy uses (the oracle's matrix products)."""
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max((i.get("num_threads", 1) for i in libs), default=1)
        blas = f"{libs[0].get('internal_api', '?')} {libs[0].get('version', '')}".strip() if libs else "unknown"
        return int(cores), blas
    except Exception:
        return os.cpu_count() or 1, "unknown"


def cpu_block_prefill(w, wts, x):
    """The oracle (numpy float64) on a whole single-block prefill workload: tokens/s."""
    import numpy as np
    import torch
    from oracle import block as ob
    S, B = w.prefill_len, w.batch
    W = {k: v.to(torch.float64).numpy() for k, v in wts.items()}
    xs = x[:, :S].to(torch.float64).numpy()
    ck = np.zeros((B, S, w.n_kv_heads, w.head_dim))
    cv = np.zeros_like(ck)
    t0 = time.perf_counter()
    ob.block_forward(xs, W, ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)
    dt = time.perf_counter() - t0
    return {"tokens_per_s": round(B * S / dt, 1), "seconds": round(dt, 2),
            "sample": f"the whole {w.name} workload ({B} x {S}-token prefill), numpy float64"}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_decode_step_us(w, wts, x, cache_k, cache_v, p0):
    """The oracle (numpy float64) on one one-token call of a decode workload: microseconds."""
    import numpy as np
    import torch
    from oracle import block as ob
    W = {k: v.to(torch.float64).numpy() for k, v in wts.items()}
    ck = np.array(cache_k, dtype=np.float64)
    cv = np.array(cache_v, dtype=np.float64)
    xs = x.to(torch.float64).numpy()
    t0 = time.perf_counter()
    ob.block_forward(xs, W, ck, cv, p0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)
    return (time.perf_counter() - t0) * 1e6


def bench_tiny(dev, cpu):
    """The tiny fp32 workload (dim 256, GQA 8/2, one 64-token prompt, then 16 one-token
    calls): launch-latency bound, so absolute microseconds per call, and the
    one-token call replayed from a HIP graph (its GPU-side time)."""
    import numpy as np
    import torch
    import workloads as wl
    from decoder_block_amd.runner import BlockRunner, model_args_for
    w = wl.WORKLOADS[1]
    wts = wl.block_weights(w)
    r = BlockRunner(model_args_for(w), wts, torch.float32, dev)
    x = wl.activations(w).to(dev)
    S = w.prefill_len
    xp = x[:, :S].contiguous()
    xs = [x[:, S + t:S + t + 1].contiguous() for t in range(w.decode_steps)]
    for _ in range(10):                        # untimed: code loading, clocks
        r.forward(xp, 0)
    torch.cuda.synchronize()
    pre = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        r.forward(xp, 0)
        e1.record()
        torch.cuda.synchronize()
        pre.append(e0.elapsed_time(e1) * 1e3)
    dec = []
    for t, xt in enumerate(xs):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        r.forward(xt, S + t)
        e1.record()
        torch.cuda.synchronize()
        dec.append(e0.elapsed_time(e1) * 1e3)
    # The first one-token call again, replayed from a captured HIP graph: the step's
    # GPU-side time without the host's per-launch cost (each replay rewrites the
    # same cache row with the same values, so every replay must match the eager call).
    og = torch.empty_like(xs[0])
    r.reserve(1, 1, S)
    eager = r.forward(xs[0], S).clone()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        r.forward(xs[0], S, og)
    gdec = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        gdec.append(e0.elapsed_time(e1) * 1e3)
        if not torch.equal(og, eager):
            raise RuntimeError("tiny-f32: a graph replay of the one-token call differs from the eager call")
    del gr
    res = {"prefill_us_median": round(pct(pre, 0.5), 1), "decode_step_us_median": round(pct(dec, 0.5), 1),
           "decode_steps": len(dec), "graph_decode_step_us_median": round(pct(gdec, 0.5), 1), "dtype": "f32"}
    if cpu:
        from oracle import block as ob
        W = {k: v.to(torch.float64).numpy() for k, v in wts.items()}
        xc = x.cpu().to(torch.float64).numpy()
        shape = (1, w.max_seq_len, w.n_kv_heads, w.head_dim)
        ck, cv = np.zeros(shape), np.zeros(shape)
        t0 = time.perf_counter()
        ob.block_forward(xc[:, :S], W, ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)
        t1 = time.perf_counter()
        ob.block_forward(xc[:, S:S + 1], W, ck, cv, S, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)
        t2 = time.perf_counter()
        res["cpu_oracle_prefill_us"] = round((t1 - t0) * 1e6, 1)
        res["cpu_oracle_decode_step_us"] = round((t2 - t1) * 1e6, 1)
    return res


def stack_oracle_sample(w):
    """The oracle on a bounded sample of the 32-layer workload: sequence 0 of 64,
    layers 0 and 1 (weights generated and upcast layer by layer), its 2048-token
    prompt and then one one-token call.  Returns the cpu_baseline object in the
    headline's unit (prefill tokens/s per block) plus the decode step scaled to
    32 layers."""
    import numpy as np
    import torch
    import workloads as wl
    from oracle import block as ob
    emb, _, _ = wl.stack_tensors(w)
    tok = wl.prompt_tokens(w)[0:1]
    h = emb[tok].to(torch.float64).numpy()                 # [1, S, D]
    hd = emb[tok[:, -1:]].to(torch.float64).numpy()        # stand-in for the next token's row
    S = w.prefill_len
    shape = (1, S + 1, w.n_kv_heads, w.head_dim)
    t_pre = t_dec = 0.0
    layers = 2
    for l in range(layers):
        W = {k: v.to(torch.float64).numpy() for k, v in wl.block_weights(w, l).items()}
        ck, cv = np.zeros(shape), np.zeros(shape)
        t0 = time.perf_counter()
        h = ob.block_forward(h, W, ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)
        t1 = time.perf_counter()
        hd = ob.block_forward(hd, W, ck, cv, S, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)
        t2 = time.perf_counter()
        t_pre += t1 - t0
        t_dec += t2 - t1
    cores, blas = blas_threads()
    return {"value": round(S * layers / t_pre, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"sequence 0 of {w.batch} ({S}-token prompt), layers 0-1 of {w.n_layers}, numpy float64: "
                      f"{t_pre:.1f} s of prefill; prefill tokens/s per block = {S} tokens x {layers} blocks / that "
                      f"time (embedding and output projection not included)",
            "decode_ms_per_step_scaled_to_32_layers": round(t_dec * w.n_layers / layers * 1e3, 1),
            "blas": blas, "cpu": cpu_model()}


def stack_layer_weights(w):
    """The seeded weights of every layer, generated on host threads (torch's
    generators release the GIL; each layer's draws are independent of the order)."""
    import concurrent.futures as cf
    import workloads as wl
    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        return list(ex.map(lambda l: wl.block_weights(w, l), range(w.n_layers)))


def bench_stack(dev, steps, warmup, decode_steps):
    """The headline: 32 layers + embedding + LM head.  ``steps`` timed prefill calls of
    64 x 2048 prompts (after ``warmup`` untimed ones), one more with stage events on
    every layer, then ``decode_steps`` greedy one-token steps (eager, replayed from a
    HIP graph, and sampled with temperature + top-p from a graph)."""
    import torch
    import workloads as wl
    from decoder_block_amd.model import StackRunner
    from decoder_block_amd.runner import model_args_for
    w = wl.WORKLOADS[5]
    log(f"workload {w.name}: generating {w.n_layers} layers")
    layers = stack_layer_weights(w)
    emb, norm_w, w_out = wl.stack_tensors(w)
    stack = StackRunner(model_args_for(w), lambda l: layers[l], emb, norm_w, w_out, torch.bfloat16, dev)
    del layers, emb, w_out
    B, S = w.batch, w.prefill_len
    decode_steps = min(decode_steps, w.decode_steps)
    prompt = wl.prompt_tokens(w).to(dev)
    out = torch.empty(decode_steps + 1, B, dtype=torch.int32, device=dev)
    logits = torch.empty(B, w.vocab_size, dtype=torch.float32, device=dev)
    log(f"stack prefill: {warmup} warm-up + {steps} timed steps")
    for _ in range(warmup):
        stack.forward(prompt, 0, logits, out[0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stack.forward(prompt, 0, logits, out[0])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    log(f"stack prefill {wall * 1e3:.1f} ms")
    # per-stage durations of every layer from HIP events recorded on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(w.n_layers)]
    stack.forward(prompt, 0, logits, out[0], layer_events=evs)
    torch.cuda.synchronize()
    stage_ms = [sum(e[i - 1].elapsed_time(e[i]) for e in evs) / w.n_layers for i in range(1, 8)]
    # greedy decode from the prefilled caches, eager
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    for t in range(decode_steps):
        stack.forward(out[t].view(B, 1), S + t, logits, out[t + 1])
    e[1].record()
    torch.cuda.synchronize()
    dec = e[0].elapsed_time(e[1]) / decode_steps
    log(f"stack decode {dec:.3f} ms/step")
    # the same steps replayed from one captured HIP graph (position held on the device)
    stack.forward(prompt, 0, logits, out[0])
    tok = out[0].clone()
    pos = torch.full((1,), S, dtype=torch.int32, device=dev)
    max_pos = S + decode_steps - 1                       # the last position a timed step writes
    stack.decode_step_at(tok, pos, max_pos, logits)      # eager first step (loads the kernels)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack.decode_step_at(tok, pos, max_pos, logits)
    pos.fill_(S)
    tok.copy_(out[0])
    torch.cuda.synchronize()
    e[0].record()
    for _ in range(decode_steps):
        graph.replay()
    e[1].record()
    torch.cuda.synchronize()
    dec_g = e[0].elapsed_time(e[1]) / decode_steps
    log(f"stack decode from a HIP graph {dec_g:.3f} ms/step")
    del graph
    # the same loop sampling with temperature 0.8 and top-p 0.95 (the walkthrough's
    # defaults); fresh uniforms are copied in between replays, as generate() does
    pos.fill_(S)
    tok.copy_(out[0])
    gu = torch.Generator(device=dev).manual_seed(7)
    us = torch.rand(decode_steps + 1, B, generator=gu, device=dev)
    ubuf = us[0].clone()
    stack.decode_step_at(tok, pos, max_pos, logits, 0.8, 0.95, ubuf)      # eager first step
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack.decode_step_at(tok, pos, max_pos, logits, 0.8, 0.95, ubuf)
    pos.fill_(S)
    tok.copy_(out[0])
    torch.cuda.synchronize()
    e[0].record()
    for t in range(decode_steps):
        ubuf.copy_(us[t + 1])
        graph.replay()
    e[1].record()
    torch.cuda.synchronize()
    dec_s = e[0].elapsed_time(e[1]) / decode_steps
    log(f"stack sampled decode from a HIP graph {dec_s:.3f} ms/step")
    del graph
    # top-p sampling of the last step's logits alone
    g = torch.Generator(device=dev).manual_seed(5)
    uni = torch.rand(20, B, generator=g, device=dev)
    from decoder_block_amd import _lib as L
    L.llama_sample_top_p(logits, out[0], B, w.vocab_size, 0.8, 0.95, uni[0])
    torch.cuda.synchronize()
    e[0].record()
    for i in range(20):
        L.llama_sample_top_p(logits, out[0], B, w.vocab_size, 0.8, 0.95, uni[i])
    e[1].record()
    torch.cuda.synchronize()
    samp = e[0].elapsed_time(e[1]) / 20
    work = stage_work(w, B, S, 0)
    stages = {}
    for name, ms in zip(STAGES, stage_ms):
        kind, amount = work[name]
        if kind == "mfma":
            ach = amount / (ms * 1e-3) / 1e12
            stages[name] = {"ms": round(ms, 4), "tflops": round(ach, 1), "mfma_frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = amount / (ms * 1e-3) / 1e9
            stages[name] = {"ms": round(ms, 4), "gbs": round(ach, 1), "hbm_frac": round(ach / PEAK_HBM_GBS, 4)}
    res = {"wall_s": wall, "stage_ms": stage_ms, "work": work,
           "prefill_ms": round(wall * 1e3, 2), "stack_prefill_tokens_per_s": round(B * S / wall, 1),
           "layer_stages": stages,
           "decode_ms_per_step": round(dec, 3), "decode_tokens_per_s": round(B / dec * 1e3, 1),
           "graph_decode_ms_per_step": round(dec_g, 3), "graph_decode_tokens_per_s": round(B / dec_g * 1e3, 1),
           "graph_sampled_decode_ms_per_step": round(dec_s, 3),
           "graph_sampled_decode_tokens_per_s": round(B / dec_s * 1e3, 1),
           "decode_steps_timed": decode_steps, "decode_positions": [S, S + decode_steps - 1], "batch": B,
           "prompt": S, "layers": w.n_layers, "top_p_sampling_us": round(samp * 1e3, 1)}
    del stack
    torch.cuda.empty_cache()
    return w, res


def bench_tp_share(dev, flush, reps):
    """One GPU's share of the 70B-shaped batch-32 decode step under 8-way tensor
    parallelism (heads split by kv head, FFN columns by eighths), at its real
    shapes: decode attention over one kv head and its 8 query heads (32 x 4097
    cached positions), and the SwiGLU FFN with 3584 hidden columns.  These two
    carry 87 % of the share's bytes; the QKV and wo shares (21 and 17 MB) and the
    two all-reduces per block are not timed here.  Each rep follows a MALL flush."""
    import torch
    from decoder_block_amd import _lib as L
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    B, T, H, Hkv, d, D, F = 32, 4097, 8, 1, 128, 8192, 3584
    args = L.ModelArgs(dim=H * d, n_layers=1, n_heads=H, n_kv_heads=Hkv, vocab_size=-1, multiple_of=256,
                       ffn_dim_multiplier=None, norm_eps=1e-5, rope_theta=5e5, max_batch_size=B, max_seq_len=T)
    ck = torch.randn(B, T, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    cv = torch.randn(B, T, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    q = torch.randn(B, 1, H, d, generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn(B, 1, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn(B, 1, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    o = torch.empty(B, 1, H * d, dtype=torch.bfloat16, device=dev)
    nba = L.llama_attn_decode_workspace_size(args, B, T - 1)
    wsa = torch.empty(max(nba, 256), dtype=torch.uint8, device=dev)
    x = torch.randn(B, D, generator=g, device=dev).to(torch.bfloat16)
    w1, w3 = ((torch.randn(F, D, generator=g, device=dev) * 0.02).to(torch.bfloat16) for _ in range(2))
    w2 = (torch.randn(D, F, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    y = torch.empty(B, D, dtype=torch.bfloat16, device=dev)
    nbf = L.llama_ffn_workspace_size(B, D, F, L.LLAMA_BF16)
    wsf = torch.empty(max(nbf, 256), dtype=torch.uint8, device=dev)
    calls = {
        "attention": (lambda: L.llama_gqa_attn_decode(q, k, v, ck, cv, o, args, B, T - 1, wsa, nba),
                      2 * B * T * Hkv * d * 2),
        "ffn": (lambda: L.llama_swiglu_ffn(x, w1, w3, w2, y, B, D, F, wsf, nbf), 3 * F * D * 2),
    }
    res = {}
    for name, (call, nbytes) in calls.items():
        call()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            flush_mall(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        med = sorted(t)[len(t) // 2]
        gbs = nbytes / (med * 1e-3) / 1e9
        res[name] = {"us_median": round(med * 1e3, 2), "us_p10": round(pct(t, 0.1) * 1e3, 2),
                     "us_p90": round(pct(t, 0.9) * 1e3, 2), "mbytes": round(nbytes / 1e6, 1),
                     "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    res["shapes"] = {"batch": B, "positions": T, "q_heads": H, "kv_heads": Hkv, "head_dim": d, "dim": D,
                     "ffn_hidden": F}
    return res


SECTIONS = ("stack", "llama7b", "llama3_8b", "llama2_70b", "tiny")


def bench_llama7b(dev, a, cpu):
    """The LLaMA-7B-shaped block prefill (batch 4 x 2048, MHA): per-stage times and
    the dual w1/w3 GEMM's fraction of the MFMA roofline at M = 8192."""
    import torch
    import workloads as wl
    log("workload llama7b-block-prefill: generating inputs")
    w2, wts2, r2 = make_runner(2, dev)
    x2 = wl.activations(w2).to(dev)
    tokens = w2.batch * w2.prefill_len
    wall, stage_ms = time_prefill(r2, x2, a.steps, a.warmup)
    work = stage_work(w2, w2.batch, w2.prefill_len, 0)
    stages = {}
    for name, ms in zip(STAGES, stage_ms):
        kind, amount = work[name]
        if kind == "mfma":
            ach = amount / (ms * 1e-3) / 1e12
            stages[name] = {"ms": round(ms, 4), "tflops": round(ach, 1), "mfma_frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = amount / (ms * 1e-3) / 1e9
            stages[name] = {"ms": round(ms, 4), "gbs": round(ach, 1), "hbm_frac": round(ach / PEAK_HBM_GBS, 4)}
    total = sum(work[n][1] for n in STAGES if work[n][0] == "mfma")
    res = {"tokens_per_s": round(tokens / wall, 1), "ms": round(wall * 1e3, 4),
           "block_tflops": round(total / wall / 1e12, 1), "block_mfma_frac": round(total / wall / 1e12 /
                                                                                   PEAK_BF16_TFLOPS, 4),
           "stages": stages, "w1w3_traffic_bytes": kernel_traffic("w1w3_swiglu_llama7b")}
    del r2
    torch.cuda.empty_cache()
    if cpu:
        res["cpu_oracle"] = cpu_block_prefill(w2, wts2, wl.activations(w2))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps (stack prefill calls; block prefill calls)")
    # (10 by default: after set-up, 3 untimed calls left the first timed window
    # 2-8 % slow at identical kernel times)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=16,
                    help="timed one-token calls of the single-block decode workloads")
    ap.add_argument("--stack-decode-steps", type=int, default=256,
                    help="greedy one-token steps of the 32-layer stack (the workload's 256)")
    ap.add_argument("--sections", default=",".join(SECTIONS),
                    help="comma-separated subset of " + ",".join(SECTIONS) + " (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (scales rocprofv3 FETCH/WRITE_SIZE)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported (this build has no multi-GPU "
              f"path)", file=sys.stderr)
        sys.exit(2)
    sections = [x for x in a.sections.split(",") if x]
    unknown = [x for x in sections if x not in SECTIONS]
    if unknown:
        print(f"unknown sections {unknown}; choose from {SECTIONS}", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cpu = not a.no_cpu_baseline
    if a.calibration_copy:
        src = torch.ones(1 << 29, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    extra = {}
    value = wall = roofline = cpu_base = None
    w5 = wl.WORKLOADS[5]
    # ---------------------------------------------------------------- headline: the 32-layer stack
    if "stack" in sections:
        w5, st = bench_stack(dev, a.steps, a.warmup, a.stack_decode_steps)
        wall = st.pop("wall_s")
        stage_ms, work = st.pop("stage_ms"), st.pop("work")
        value = w5.batch * w5.prefill_len * w5.n_layers / wall
        dom = "w1w3_swiglu"
        dom_ms = stage_ms[STAGES.index(dom)]
        dom_ach = work[dom][1] / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": "gemm_bf16_dma<256x256x64, 8 waves, DUAL, EpiSwiGLU> (w1/w3 + SwiGLU, "
                    "M = 131072, N = 2 x 14336, K = 4096)", "achieved": round(dom_ach, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(dom_ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": kernel_traffic("w1w3_swiglu_llama3_8b_stack"), "kernel_ms": round(dom_ms, 4),
                    "flops_per_launch": work[dom][1]}
        extra["llama3_8b_stack"] = st
        if cpu:
            log("cpu oracle: bounded sample of the 32-layer stack")
            cpu_base = stack_oracle_sample(w5)

    if "llama7b" in sections:
        extra["llama7b_block_prefill"] = bench_llama7b(dev, a, cpu)

    flush = None
    if "llama3_8b" in sections or "llama2_70b" in sections:
        flush = torch.zeros(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    if "llama3_8b" in sections:
        # ------------------------------------------------------------ 8B-shaped prefill 8192 + decode
        log("workload llama3-8b-block: prefill 8192 then decode steps")
        w3, wts3, r3 = make_runner(3, dev)
        x3 = wl.activations(w3).to(dev)
        S3 = w3.prefill_len
        xp = x3[:, :S3].contiguous()
        # (the same warm-up as the headline: one call measured 8 % slow right after set-up)
        wall3, stage3 = time_prefill(r3, xp, a.steps, a.warmup)
        work3 = stage_work(w3, 1, S3, 0)
        att = work3["attention"][1] / (stage3[2] * 1e-3) / 1e12
        pre3 = {"tokens_per_s": round(S3 / wall3, 1), "ms": round(wall3 * 1e3, 3),
                "attention_ms": round(stage3[2], 4), "attention_tflops": round(att, 1),
                "attention_mfma_frac": round(att / PEAK_BF16_TFLOPS, 4),
                "gemm_mfma_frac": round(sum(work3[n][1] for n in ("qkv_rope_append", "wo_residual", "w1w3_swiglu",
                                                                   "w2_residual")) /
                                        (sum(stage3[i] for i in (1, 3, 5, 6)) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        # the same 8192-token prompt fed in 4 chunks of 2048 (each chunk attends to the cached prefix)
        wallc = time_chunked_prefill(r3, xp, 2048, max(3, a.steps // 2), a.warmup)
        pre3["chunked_4x2048_tokens_per_s"] = round(S3 / wallc, 1)
        pre3["chunked_4x2048_ms"] = round(wallc * 1e3, 3)
        nd = min(a.decode_steps, w3.decode_steps)
        xs = [x3[:, S3 + t:S3 + t + 1].contiguous() for t in range(nd)]
        tot, st = time_decode(r3, xs, [S3 + t for t in range(nd)], flush)
        wb, kvb = decode_bytes(w3, 1, S3 + nd // 2)
        attn_gbs = kvb / (st[2] * 1e-3) / 1e9
        dec3 = {"step_us_mean": round(1e3 * sum(tot) / len(tot), 2),
                "step_us_median": round(1e3 * sorted(tot)[len(tot) // 2], 2),
                "step_us_p10": round(1e3 * pct(tot, 0.1), 2), "step_us_p90": round(1e3 * pct(tot, 0.9), 2),
                "attention_us": round(st[2] * 1e3, 2), "attention_gbs": round(attn_gbs, 1),
                "attention_hbm_frac": round(attn_gbs / PEAK_HBM_GBS, 4),
                "step_gbs": round((wb + kvb) / (sum(tot) / len(tot) * 1e-3) / 1e9, 1),
                "stage_us": {n: round(v * 1e3, 2) for n, v in zip(STAGES, st)},
                "steps_timed": nd, "positions": [S3, S3 + nd - 1]}
        del r3
        torch.cuda.empty_cache()
        if cpu:
            import numpy as np
            shape3 = (1, S3 + 1, w3.n_kv_heads, w3.head_dim)
            x3d = wl.activations(w3)[:, S3:S3 + 1].contiguous()
            dec3["cpu_oracle_step_us"] = round(cpu_decode_step_us(w3, wts3, x3d, np.zeros(shape3), np.zeros(shape3),
                                                                  S3), 1)
            dec3["cpu_oracle_note"] = ("oracle, numpy float64, one call at position 8192 over a zero cache of the "
                                       "same shape (its cost depends on the shape only)")
        extra["llama3_8b_prefill_8192"] = pre3
        extra["llama3_8b_decode"] = dec3
    if "llama2_70b" in sections:
        # ------------------------------------------------------------ 70B-shaped batch-32 decode
        log("workload llama2-70b-block-decode: batch 32 at position 4096")
        w4 = wl.WORKLOADS[4]
        cache = wl.prefilled_cache(w4)
        w4, wts4, r4 = make_runner(4, dev, cache=cache)
        x4 = wl.activations(w4).to(dev)
        p0 = w4.cache_prefill
        tot4 = []
        st4 = [0.0] * 7
        for _ in range(max(a.decode_steps, 3)):
            # the same token at the same position each rep: the append rewrites identical rows
            t, s_ = time_decode(r4, [x4], [p0], flush)
            tot4 += t
            st4 = [u + v for u, v in zip(st4, s_)]
        n4 = len(tot4)
        st4 = [u / n4 for u in st4]
        wb4, kvb4 = decode_bytes(w4, w4.batch, p0 + 1)
        attn4 = kvb4 / (st4[2] * 1e-3) / 1e9
        dec4 = {"step_us_mean": round(1e3 * sum(tot4) / n4, 2),
                "step_us_median": round(1e3 * sorted(tot4)[n4 // 2], 2),
                "step_us_p10": round(1e3 * pct(tot4, 0.1), 2), "step_us_p90": round(1e3 * pct(tot4, 0.9), 2),
                "attention_us": round(st4[2] * 1e3, 2), "attention_gbs": round(attn4, 1),
                "attention_hbm_frac": round(attn4 / PEAK_HBM_GBS, 4),
                "step_gbs": round((wb4 + kvb4) / (sum(tot4) / n4 * 1e-3) / 1e9, 1),
                "step_hbm_frac": round((wb4 + kvb4) / (sum(tot4) / n4 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "stage_us": {n: round(v * 1e3, 2) for n, v in zip(STAGES, st4)}}
        del r4
        torch.cuda.empty_cache()
        log("workload llama2-70b decode, one GPU's share under 8-way tensor parallelism")
        dec4["tp8_share"] = bench_tp_share(dev, flush, max(a.decode_steps, 3))
        if cpu:
            log("cpu oracle: one decode step of the 70B-shaped workload")
            c4k, c4v = (c.to(torch.float32).numpy() for c in cache)
            dec4["cpu_oracle_step_us"] = round(cpu_decode_step_us(w4, wts4, wl.activations(w4), c4k, c4v, p0), 1)
            dec4["cpu_oracle_note"] = "oracle, numpy float64, one call over the same seeded cache (host cores)"
        extra["llama2_70b_decode_b32"] = dec4
    del flush
    torch.cuda.empty_cache()
    if "tiny" in sections:
        log("workload tiny-f32: 64-token prefill, then one-token calls")
        extra["tiny_f32"] = bench_tiny(dev, cpu)

    line = {
        "metric": METRIC, "value": round(value, 1) if value is not None else None, "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(wall * 1e3, 3) if wall is not None else None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random token ids, N(0,0.02) weights, unit RMSNorm weights)",
        "config": {"workload": w5.name, "layers": w5.n_layers, "dim": w5.dim, "n_heads": w5.n_heads,
                   "n_kv_heads": w5.n_kv_heads, "ffn_hidden": w5.ffn_hidden, "vocab": w5.vocab_size,
                   "batch": w5.batch, "seq_len": w5.prefill_len, "decode_steps": a.stack_decode_steps,
                   "value_is": "prefill tokens/s per block = batch x seq_len x layers / prefill step time",
                   "parallelism": "none (1 GPU)", "sections": sections},
        "roofline": roofline,
        "cpu_baseline": cpu_base,
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
