"""The 32-layer Llama-3-8B-shaped stack (embedding, 32 blocks, final RMSNorm,
output projection of the last position, greedy argmax fed back on the device).

Parity is checked layer by layer with the oracle driving every input: the
oracle runs its own float64 chain through all 32 layers on a prompt prefix
(and one decode step), and each GPU layer receives the oracle's layer input
(rounded to bf16) and is compared with the oracle's layer output.  At the
stack's real shape (64 sequences x 2048 tokens, then one batch-64 decode step,
and the output projection over 64 x 128256 logits) layers 0 and 31 are
compared with the oracle on sampled sequences.  No GPU result is fed to the
oracle.  The full workload (batch 64 x 2048-token prompts, 256 greedy steps)
then runs end to end on the GPU, where the greedy feedback is checked exactly
against each step's logits.

Every RMSNorm weight here (both norms of each layer and the final norm) is drawn
2^k, k uniform in {-1, 0, 1}, distinct per norm and layer, so that a swapped,
dropped or misindexed gain in any fused normalisation changes the result, while
x * g stays exact in bf16: with 1 + N(0, 0.2^2) gains the rounding of x * g alone
costs layer 0 (whose input is the N(0, 0.02) embedding rows) about 4.6e-3 of
relative Frobenius error, most of the 1e-2 budget.  The per-block tests cover
that rounding with 1 + N(0, 0.2^2) gains.  The workload's other tensors are
those of the 32-layer Llama-3-8B-shaped configuration.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from decoder_block_amd import _lib as L
from decoder_block_amd.model import StackRunner
from decoder_block_amd.runner import BlockRunner, model_args_for
from oracle import block as ob
from tests.gpu_util import check, errors, f64, need_gpu

pytestmark = pytest.mark.gpu

W5 = wl.WORKLOADS[5].scaled(norm_gains="pow2")


@pytest.fixture(scope="module")
def host_weights():
    import concurrent.futures as cf
    print(f"case {W5.name}: generating {W5.n_layers} layers of seeded weights", flush=True)
    with cf.ThreadPoolExecutor(8) as ex:     # torch's generators release the GIL
        layers = list(ex.map(lambda l: wl.block_weights(W5, l), range(W5.n_layers)))
    emb, norm_w, w_out = wl.stack_tensors(W5)
    return layers, emb, norm_w, w_out


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)


def test_stack_layers_follow_the_oracle_chain(host_weights):
    dev = need_gpu()
    layers, emb, norm_w, w_out = host_weights
    P = 96                                   # prompt prefix evaluated by the oracle
    w = W5
    print(f"case {w.name}: oracle-driven per-layer parity, prefix {P} + 1 decode step", flush=True)
    args = model_args_for(w, max_batch=1, max_seq=P + 1)
    stack = StackRunner(args, lambda l: layers[l], emb, norm_w, w_out, torch.bfloat16, dev)
    prompt = wl.prompt_tokens(w)[:1, :P + 1]         # row 0; token P is the decode-step input
    tok = prompt.numpy()
    # oracle chain (float64) from the embedding rows
    h = f64(emb)[tok[:, :P]]
    hd = f64(emb)[tok[:, P:P + 1]]
    worst = 0.0
    shape = (1, P + 1, w.n_kv_heads, w.head_dim)
    for l in range(w.n_layers):
        W = {k: v.to(torch.float64).numpy() for k, v in layers[l].items()}
        ck, cv = np.zeros(shape), np.zeros(shape)
        h_next = ob.block_forward(h, W, ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)
        hd_next = ob.block_forward(hd, W, ck, cv, P, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)
        r = stack.layers[l]
        got = r.forward(_bf16(h).to(dev), 0)
        got_d = r.forward(_bf16(hd).to(dev), P)
        torch.cuda.synchronize()
        e = check(got, h_next, "bf16", f"layer {l} prefill")
        ed = check(got_d, hd_next, "bf16", f"layer {l} decode step")
        worst = max(worst, e["relf"], ed["relf"])
        h, hd = h_next, hd_next
    print(f"[parity] worst per-layer relF {worst:.3e}", flush=True)
    # final RMSNorm + output projection + greedy token from the oracle's last hidden state
    for name, last in (("prefill", h[:, -1]), ("decode", hd[:, -1])):
        ref = ob.linear(ob.rms_norm(last, f64(norm_w), w.norm_eps), f64(w_out))
        logits = torch.empty(1, w.vocab_size, dtype=torch.float32, device=dev)
        nxt = torch.empty(1, dtype=torch.int32, device=dev)
        nb = L.llama_lm_head_workspace_size(1, w.dim, w.vocab_size, L.LLAMA_BF16)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        L.llama_lm_head_argmax(_bf16(last).to(dev), w.dim, stack.norm_w, stack.w_out, logits, nxt, 1, w.dim,
                               w.vocab_size, w.norm_eps, ws, nb)
        torch.cuda.synchronize()
        e = check(logits, ref, "bf16", f"{name} logits")
        g = int(nxt.item())
        lg = f64(logits)[0]
        assert g == int(np.argmax(lg))                               # exact on the GPU's logits
        assert ref[0, g] >= ref[0].max() - 2 * e["raw_maxabs"]        # a correct greedy token


def test_stack_full_workload_greedy_generation(host_weights):
    dev = need_gpu()
    layers, emb, norm_w, w_out = host_weights
    w = W5
    steps = w.decode_steps
    print(f"case {w.name}: B={w.batch} prompt {w.prefill_len} + {steps} greedy steps", flush=True)
    stack = StackRunner(model_args_for(w), lambda l: layers[l], emb, norm_w, w_out, torch.bfloat16, dev)
    prompt = wl.prompt_tokens(w).to(dev)
    checked = {}

    def on_step(t, logits, nxt):
        if t in (0, 1, steps // 2, steps):
            checked[t] = (f64(logits), nxt.cpu().numpy().copy())

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    out = stack.generate(prompt, steps, on_step)
    ev[1].record()
    torch.cuda.synchronize()
    print(f"[stack] prefill + {steps} steps: {ev[0].elapsed_time(ev[1]):.1f} ms (includes host checks)", flush=True)
    ids = out.cpu().numpy()
    assert ids.shape == (steps + 1, w.batch)
    assert ids.min() >= 0 and ids.max() < w.vocab_size
    for t, (lg, nxt) in checked.items():
        assert np.all(np.isfinite(lg))
        np.testing.assert_array_equal(nxt, np.argmax(lg, axis=1))   # greedy = argmax, lowest id on ties
        np.testing.assert_array_equal(ids[t], nxt)                   # and that id was fed to the next call


def test_stack_top_p_sampled_generation(host_weights):
    """Sampled generation (temperature 0.8, top_p 0.95) through the whole stack: the
    sampled ids are in range, are what the next call consumes, are reproducible for
    the same uniform numbers, and depart from greedy.  The selection kernel itself is
    checked against the oracle in test_gpu_sampling.py on seeded logits."""
    dev = need_gpu()
    layers, emb, norm_w, w_out = host_weights
    w = W5
    steps, S = 8, 128
    print(f"case {w.name}: B={w.batch} prompt {S} + {steps} sampled steps (T=0.8, top_p=0.95)", flush=True)
    stack = StackRunner(model_args_for(w), lambda l: layers[l], emb, norm_w, w_out, torch.bfloat16, dev)
    prompt = wl.prompt_tokens(w)[:, :S].contiguous().to(dev)
    g = torch.Generator(device=dev).manual_seed(99)
    uni = torch.rand(steps + 1, w.batch, generator=g, device=dev)
    a = stack.generate(prompt, steps, temperature=0.8, top_p=0.95, uniforms=uni).cpu().numpy()
    b = stack.generate(prompt, steps, temperature=0.8, top_p=0.95, uniforms=uni).cpu().numpy()
    greedy = stack.generate(prompt, steps).cpu().numpy()
    torch.cuda.synchronize()
    assert a.shape == (steps + 1, w.batch)
    assert a.min() >= 0 and a.max() < w.vocab_size
    np.testing.assert_array_equal(a, b)
    assert np.mean(a[0] != greedy[0]) > 0.5        # flat synthetic logits: sampling rarely picks the argmax
    del stack
    torch.cuda.empty_cache()


def _device_position_decode(stack, prompt, steps, temperature=0.0, top_p=0.95, uniforms=None):
    """The device-position step run eagerly (no graph): ids and logits of every step."""
    bsz, S = prompt.shape
    dev = prompt.device
    out = torch.empty(steps + 1, bsz, dtype=torch.int32, device=dev)
    logits = torch.empty(bsz, stack.vocab, dtype=torch.float32, device=dev)
    stack.forward(prompt, 0, logits, out[0])
    if temperature > 0:
        L.llama_sample_top_p(logits, out[0], bsz, stack.vocab, temperature, top_p, uniforms[0])
    tok = out[0].clone()
    pos = torch.full((1,), S, dtype=torch.int32, device=dev)
    u = torch.empty(bsz, dtype=torch.float32, device=dev)
    lg = []
    for t in range(1, steps + 1):
        if temperature > 0:
            u.copy_(uniforms[t])
        stack.decode_step_at(tok, pos, S + steps - 1, logits, temperature, top_p, u)
        out[t].copy_(tok)
        lg.append(logits.clone())
    return out, lg


@pytest.mark.parametrize("temperature", [0.0, 0.8])
def test_stack_graph_decode_replays_match_eager(host_weights, temperature):
    """generate(graph=True) captures one whole decode step (embedding, 32 layers,
    norm, output projection, token choice, position advance) in a HIP graph and
    replays it.  Every replay, with eager library work and a synchronisation
    between replays, must reproduce the same step run eagerly through the same
    device-position entry point bit for bit (ids and fp32 logits).

    The host-position path is compared with this one layer by layer in
    test_stack_decode_paths_agree_layer_by_layer."""
    dev = need_gpu()
    layers, emb, norm_w, w_out = host_weights
    w = W5
    steps, S = 10, 128
    print(f"case {w.name}: HIP-graph decode, B={w.batch} prompt {S} + {steps} steps, T={temperature}", flush=True)
    stack = StackRunner(model_args_for(w), lambda l: layers[l], emb, norm_w, w_out, torch.bfloat16, dev)
    prompt = wl.prompt_tokens(w)[:, :S].contiguous().to(dev)
    g = torch.Generator(device=dev).manual_seed(123)
    uni = torch.rand(steps + 1, w.batch, generator=g, device=dev)
    kw = dict(temperature=temperature, top_p=0.95, uniforms=uni) if temperature > 0 else {}
    scratch_x = torch.randn(w.batch, w.dim, generator=g, device=dev).to(torch.bfloat16)
    scratch_y = torch.empty_like(scratch_x)
    graph_logits = {}

    def on_step(t, logits, nxt):
        if t == 0:
            return
        graph_logits[t] = logits.clone()
        torch.cuda.synchronize()
        # eager library work between replays
        L.llama_rmsnorm(scratch_x, stack.norm_w, scratch_y, w.batch, w.dim, w.norm_eps)
        torch.cuda.synchronize()

    got = stack.generate(prompt, steps, on_step, graph=True, **kw)
    torch.cuda.synchronize()
    ref, ref_logits = _device_position_decode(stack, prompt, steps, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy())
    for t in range(1, steps + 1):
        assert torch.equal(graph_logits[t], ref_logits[t - 1]), f"step {t}: replay differs from the eager step"
    print(f"[graph] {steps} replays bit-identical to the eager device-position steps", flush=True)
    del stack
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,bound", [(64, 128 + 255), (4, 2200)])
def test_stack_decode_paths_agree_layer_by_layer(host_weights, B, bound):
    """One decode step through both one-token entry points on identical per-layer
    inputs: llama_block_forward (position passed by the host, attention split by
    the actual length) and llama_block_decode_at (position read on the device,
    splits laid out for the bound).  At batch 64 both take one split per
    (sequence, kv group) and must agree bit for bit; at batch 4 the bound of 2200
    positions lays out 14 splits where the host path uses 2, so the fp32 sums run
    in another order (and the projections take the one-to-four-token weight
    streams).  Layer l's input is the host-position path's output of layer l - 1;
    the outputs of every layer and the appended k rows must agree within the bf16
    tolerance."""
    dev = need_gpu()
    layers, emb, norm_w, w_out = host_weights
    w = W5
    S = 128
    print(f"case {w.name}: decode step at {S} through both one-token entry points, B={B}, bound {bound}",
          flush=True)
    args = model_args_for(w, max_batch=B, max_seq=bound + 1)
    stack = StackRunner(args, lambda l: layers[l], emb, norm_w, w_out, torch.bfloat16, dev)
    prompt = wl.prompt_tokens(w)[:B, :S].contiguous().to(dev)
    logits = torch.empty(B, w.vocab_size, dtype=torch.float32, device=dev)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    stack.forward(prompt, 0, logits, tok)
    D = w.dim
    need = max(L.llama_block_workspace_size(args, B, 1, bound, L.LLAMA_BF16),
               L.llama_block_workspace_size(args, B, 1, S, L.LLAMA_BF16))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    pos = torch.full((1,), S, dtype=torch.int32, device=dev)
    h = torch.empty(B, 1, D, dtype=torch.bfloat16, device=dev)
    L.llama_embedding(tok, stack.embedding, h, B, D, w.vocab_size)
    worst = 0.0
    for l, r in enumerate(stack.layers):
        a = torch.empty_like(h)
        b = torch.empty_like(h)
        L.llama_block_forward(args, r.cw, r.cache_k, r.cache_v, r.freqs, r.freqs_end, h, a, B, 1, S, ws, need)
        ka = r.cache_k[:, S].clone()
        L.llama_block_decode_at(args, r.cw, r.cache_k, r.cache_v, r.freqs, r.freqs_end, h, b, B, pos, bound, ws,
                                need)
        torch.cuda.synchronize()
        e = check(b, f64(a), "bf16", f"layer {l}: device-position vs host-position output")
        assert torch.equal(ka, r.cache_k[:, S]), f"layer {l}: the two paths appended different k rows"
        if B == 64:
            assert torch.equal(a, b), f"layer {l}: one split each, yet the outputs differ"
        worst = max(worst, e["relf"])
        h = a
    print(f"[paths] worst per-layer relF between the two one-token paths {worst:.3e}", flush=True)
    del stack
    torch.cuda.empty_cache()


def test_stack_real_shape_layers_decode_and_lm_head(host_weights):
    """The stack's own shapes: layers 0 and 31 each run a 64 x 2048 prefill (the
    M = 131072 projections, attention dispatched in cache-sized sequence groups),
    then one batch-64 decode step (64-row split-K projections with wo's reduction
    fused with ffn_norm, split decode attention over 2049 keys), and the final
    norm + output projection runs over 64 x 128256 logits.  Layer 0 receives the
    embedding rows of the workload's prompt ids, layer 31 seeded N(0, 4^2) rows
    (a deep layer's scale).  The oracle evaluates sampled sequences (each on its
    own: batch rows are independent) at sampled positions, their whole appended
    caches and their decode rows, and every logit of the output projection."""
    dev = need_gpu()
    layers, emb, norm_w, w_out = host_weights
    w = W5
    B, S, D = w.batch, w.prefill_len, w.dim
    seqs = [0, 21, 42, 63]
    rows = sorted({0, 1, 63, 64, 127, 128, 1023, 1024, S // 2 + 17, S - 2, S - 1})
    args = model_args_for(w, max_seq=S + 1)
    g = torch.Generator().manual_seed(20251)
    x_dec = (torch.randn(B, 1, D, generator=g)).to(torch.bfloat16)
    for l in (0, 31):
        if l == 0:
            x = emb[wl.prompt_tokens(w).long()]                        # [B, S, D], exact gather
        else:
            x = (4.0 * torch.randn(B, S, D, generator=g)).to(torch.bfloat16)
        print(f"case {w.name}: layer {l} at B={B} S={S}, then one decode step", flush=True)
        r = BlockRunner(args, layers[l], torch.bfloat16, dev)
        out = r.forward(x.to(dev), 0)
        out_d = r.forward(x_dec.to(dev), S)
        torch.cuda.synchronize()
        W = {k: v.to(torch.float64).numpy() for k, v in layers[l].items()}
        shape = (1, S + 1, w.n_kv_heads, w.head_dim)
        for b in seqs:
            ck, cv = np.zeros(shape), np.zeros(shape)
            xb = x[b:b + 1].to(torch.float64).numpy()
            ref = ob.block_forward(xb, W, ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta, rows=rows)
            check(out[b:b + 1, rows], ref, "bf16", f"layer {l} sequence {b} prefill rows")
            check(r.cache_k[b:b + 1, :S], ck[:, :S], "bf16", f"layer {l} sequence {b} cache_k")
            check(r.cache_v[b:b + 1, :S], cv[:, :S], "bf16", f"layer {l} sequence {b} cache_v")
            ref_d = ob.block_forward(f64(x_dec[b:b + 1]), W, ck, cv, S, w.n_heads, w.n_kv_heads, w.norm_eps,
                                     w.rope_theta)
            check(out_d[b:b + 1], ref_d, "bf16", f"layer {l} sequence {b} decode step")
            check(r.cache_k[b:b + 1, S], ck[:, S], "bf16", f"layer {l} sequence {b} appended k")
        del r, out, out_d
        torch.cuda.empty_cache()
    # final RMSNorm + output projection + greedy token over the whole batch
    print(f"case {w.name}: output projection over {B} x {w.vocab_size} logits", flush=True)
    hl = (3.0 * torch.randn(B, D, generator=g)).to(torch.bfloat16)
    gn, gw = norm_w.to(dev), w_out.to(dev)
    logits = torch.empty(B, w.vocab_size, dtype=torch.float32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    nb = L.llama_lm_head_workspace_size(B, D, w.vocab_size, L.LLAMA_BF16)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    L.llama_lm_head_argmax(hl.to(dev), D, gn, gw, logits, nxt, B, D, w.vocab_size, w.norm_eps, ws, nb)
    torch.cuda.synchronize()
    ref = ob.linear(ob.rms_norm(f64(hl), f64(norm_w), w.norm_eps), f64(w_out))
    e = check(logits, ref, "bf16", "output projection logits, 64 x 128256")
    lg = f64(logits)
    got = nxt.cpu().numpy()
    for b in range(B):
        assert got[b] == int(np.argmax(lg[b]))                        # exact on the GPU's logits
        assert ref[b, got[b]] >= ref[b].max() - 2 * e["raw_maxabs"]   # a correct greedy token
