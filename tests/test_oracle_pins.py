"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage or the mathematical fact it pins.  The last test
plants plausible mistakes into the oracle (on the CPU) and checks that some
pin catches each of them.
"""
import cmath
import math
import os

import numpy as np
import pytest

from oracle import block as ob
from oracle import brute
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = v
    return out


def _rng(seed=0):
    return np.random.default_rng(seed)


def _rand_weights(rng, D, H, Hkv, F, std=0.3):
    d = D // H
    return {
        "attention_norm": 1.0 + 0.1 * rng.standard_normal(D),
        "ffn_norm": 1.0 + 0.1 * rng.standard_normal(D),
        "wq": std * rng.standard_normal((H * d, D)),
        "wk": std * rng.standard_normal((Hkv * d, D)),
        "wv": std * rng.standard_normal((Hkv * d, D)),
        "wo": std * rng.standard_normal((D, H * d)),
        "w1": std * rng.standard_normal((F, D)),
        "w2": std * rng.standard_normal((D, F)),
        "w3": std * rng.standard_normal((F, D)),
    }


def _cache(B, T, Hkv, d):
    return np.zeros((B, T, Hkv, d)), np.zeros((B, T, Hkv, d))


# ----------------------------------------------------------------------------- widths
def test_ffn_width_rule_reproduces_stated_widths():
    g = _golden("model_shapes.txt")
    # LLaMA-7B printout: 4096 -> 11008 with multiple_of 256 and no multiplier
    assert ob.ffn_hidden_dim(int(g["llama7b_dim"]), 256, None) == int(g["llama7b_ffn"])
    assert ob.ffn_hidden_dim(256, 256, None) == 768
    assert ob.ffn_hidden_dim(4096, 1024, 1.3) == 14336
    assert ob.ffn_hidden_dim(8192, 1024, 1.3) == 28672
    for w in wl.WORKLOADS.values():
        assert ob.ffn_hidden_dim(w.dim, w.multiple_of, w.ffn_dim_multiplier) == w.ffn_hidden
    # size table: head_dim = dimension / n_heads = 128 for every LLaMA-1 size
    for row in g["size_table"].split(";"):
        _, dim, heads, _ = row.split()
        assert int(dim) // int(heads) == 128


# ----------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_unit_weight_rows_have_unit_rms():
    rng = _rng(1)
    x = rng.standard_normal((64, 256)) * rng.uniform(0.1, 10, (64, 1))
    eps = 1e-5
    y = ob.rms_norm(x, np.ones(256), eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    assert np.all(np.abs(np.sqrt(np.mean(y * y, axis=-1)) - 1) < 1e-3)


def test_rmsnorm_printed_row_statistics():
    """The printed RMSNorm row (emb_dim 10, eps 1e-8) has mean(y^2) = 1, so its unbiased
    std s and mean m obey s^2 = n/(n-1) * (1 - m^2); the oracle's rows obey the same law,
    and the printed LayerNorm row (mean 0) has s = sqrt(n/(n-1))."""
    g = _golden("rmsnorm_printed_row_stats.txt")
    n = int(g["emb_dim"])
    tol = float(g["print_rel_tol"])
    m, s = float(g["rms_mean"]), float(g["rms_std"])
    assert abs(s * s - n / (n - 1) * (1 - m * m)) / (s * s) < 3 * tol
    assert abs(float(g["ln_std"]) - math.sqrt(n / (n - 1))) < 1e-4
    rng = _rng(2)
    x = rng.standard_normal((200, n))
    y = ob.rms_norm(x, np.ones(n), float(g["rms_eps"]))
    mean = y.mean(-1)
    std = y.std(-1, ddof=1)
    np.testing.assert_allclose(std ** 2, n / (n - 1) * (1 - mean ** 2), rtol=1e-6)


def test_rmsnorm_closed_forms():
    # constant row c: c / sqrt(c^2 + eps); weight multiplies elementwise; no centring
    for c in (-3.0, 0.5, 7.0):
        y = ob.rms_norm(np.full((1, 8), c), np.arange(1, 9, dtype=float), 1e-6)
        np.testing.assert_allclose(y[0], c / math.sqrt(c * c + 1e-6) * np.arange(1, 9), rtol=1e-14)
    rng = _rng(3)
    x = rng.standard_normal((4, 32))
    np.testing.assert_allclose(ob.rms_norm(5 * x, np.ones(32), 0.0), ob.rms_norm(x, np.ones(32), 0.0), rtol=1e-13)
    # an all-positive row stays all-positive (no mean is subtracted)
    assert np.all(ob.rms_norm(np.abs(x) + 0.1, np.ones(32), 1e-6) > 0)


# ----------------------------------------------------------------------------- RoPE
def test_rope_pairing_matches_printed_view_as_complex_and_polar():
    g = _golden("torch_helpers_printed.txt")
    u = np.array([float(v) for v in g["view_as_complex_in"].split()])
    # position 0 is the identity; the pairs are (even, odd) = (real, imag)
    out0 = ob.apply_rope(u.reshape(1, 1, 1, 6), [0], 1e4).reshape(-1)
    np.testing.assert_array_equal(out0[0::2], [float(v) for v in g["view_as_complex_out_re"].split()])
    np.testing.assert_array_equal(out0[1::2], [float(v) for v in g["view_as_complex_out_im"].split()])
    # table entry = cos + i sin (polar): theta_0 = 1, so entry [p, 0] = e^{ip};
    # the printed polar(1, pi/2) real part is cos(pi/2) in float64
    tab = ob.freqs_cis(int(g["freqs_dim"]), int(g["freqs_end"]), 1e4)
    assert tab.shape == (int(g["freqs_rows"]), int(g["freqs_cols"]))
    assert np.all(tab[0] == 1 + 0j)
    for p in range(10):
        assert abs(tab[p, 0] - cmath.exp(1j * p)) < 1e-15
    assert abs(math.cos(math.pi / 2) - float(g["polar_re"])) < 1e-20


def test_rope_hand_values_d4():
    """d = 4, theta = 1e4: theta_i = 1, 1e4^(-1/2) = 0.01; u = (1,0,1,0) at p = 3."""
    out = ob.apply_rope(np.array([1.0, 0, 1.0, 0]).reshape(1, 1, 1, 4), [3], 1e4).reshape(-1)
    np.testing.assert_allclose(out, [math.cos(3), math.sin(3), math.cos(0.03), math.sin(0.03)], atol=1e-15)
    # the second slot rotates (0,1) -> (-sin, cos): sign of the 2x2 rotation
    out = ob.apply_rope(np.array([0.0, 1.0, 0, 1.0]).reshape(1, 1, 1, 4), [3], 1e4).reshape(-1)
    np.testing.assert_allclose(out, [-math.sin(3), math.cos(3), -math.sin(0.03), math.cos(0.03)], atol=1e-15)
    # theta = 5e5, d = 8: theta_3 = 5e5^(-6/8)
    out = ob.apply_rope(np.array([0, 0, 0, 0, 0, 0, 1.0, 0]).reshape(1, 1, 1, 8), [1000], 5e5).reshape(-1)
    a = 1000 * 5e5 ** (-0.75)
    np.testing.assert_allclose(out[6:], [math.cos(a), math.sin(a)], atol=1e-13)


def test_rope_equals_complex_multiply():
    rng = _rng(4)
    d, S = 16, 9
    u = rng.standard_normal((2, S, 3, d))
    pos = list(range(100, 100 + S))
    out = ob.apply_rope(u, pos, 5e5)
    z = u[..., 0::2] + 1j * u[..., 1::2]
    tab = ob.freqs_cis(d, 200, 5e5)[pos]
    rz = z * tab[None, :, None, :]
    np.testing.assert_allclose(out[..., 0::2], rz.real, atol=1e-13)
    np.testing.assert_allclose(out[..., 1::2], rz.imag, atol=1e-13)


def test_rope_norm_and_relative_position():
    rng = _rng(5)
    d = 32
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, 1, d))
    for p in (0, 1, 77, 8319):
        np.testing.assert_allclose(np.linalg.norm(ob.apply_rope(q, [p], 1e4)), np.linalg.norm(q), rtol=1e-13)
    np.testing.assert_array_equal(ob.apply_rope(q, [0], 1e4), q)
    for (m, n) in ((5, 2), (100, 40), (3000, 2999)):
        ref = np.sum(ob.apply_rope(q, [m], 1e4) * ob.apply_rope(k, [n], 1e4))
        for shift in (1, 17, 1000):
            got = np.sum(ob.apply_rope(q, [m + shift], 1e4) * ob.apply_rope(k, [n + shift], 1e4))
            assert abs(got - ref) < 1e-9 * max(1, abs(ref))
    # the inner product is Re(sum q~ conj(k~) e^{i(m-n)theta_i})
    m, n = 50, 20
    qz = q[..., 0::2] + 1j * q[..., 1::2]
    kz = k[..., 0::2] + 1j * k[..., 1::2]
    th = np.array([1e4 ** (-2 * i / d) for i in range(d // 2)])
    expect = np.real(np.sum(qz * np.conj(kz) * np.exp(1j * (m - n) * th)))
    got = np.sum(ob.apply_rope(q, [m], 1e4) * ob.apply_rope(k, [n], 1e4))
    assert abs(got - expect) < 1e-12


def test_rope_interleaved_equals_half_split_after_row_permutation():
    """HF rotate_half RoPE (pairs i, i+d/2, emb = cat(freqs, freqs)) on per-head rows
    permuted [0,2,4,..,1,3,5,..] gives the same vector, permuted the same way."""
    rng = _rng(6)
    d = 16
    u = rng.standard_normal((1, 4, 2, d))
    pos = [0, 3, 9, 1000]
    perm = np.r_[np.arange(0, d, 2), np.arange(1, d, 2)]
    inv = 1.0 / (1e4 ** (np.arange(0, d, 2) / d))
    freqs = np.outer(pos, inv)
    emb = np.concatenate([freqs, freqs], axis=-1)
    cos, sin = np.cos(emb)[None, :, None, :], np.sin(emb)[None, :, None, :]
    up = u[..., perm]
    rot_half = np.concatenate([-up[..., d // 2:], up[..., :d // 2]], axis=-1)
    hf = up * cos + rot_half * sin
    np.testing.assert_allclose(ob.apply_rope(u, pos, 1e4)[..., perm], hf, atol=1e-13)


# ----------------------------------------------------------------------------- attention
def test_softmax_rows_sum_to_one_and_mask():
    rng = _rng(7)
    B, S, H, d, p0 = 2, 6, 4, 8, 3
    q = rng.standard_normal((B, S, H, d))
    keys = rng.standard_normal((B, p0 + S, H, d))
    P = ob.attention_probs(q, keys, p0)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=1e-14)
    for s in range(S):
        assert np.all(P[:, :, s, p0 + s + 1:] == 0)
        assert np.all(P[:, :, s, :p0 + s + 1] > 0)
    # single-token call: no mask, every cached key visible
    P1 = ob.attention_probs(q[:, :1], keys, p0 + S - 1)
    assert np.all(P1 > 0)


def test_equal_keys_give_mean_of_visible_values():
    rng = _rng(8)
    B, S, H, Hkv, d, p0 = 1, 5, 4, 2, 8, 2
    T = p0 + S
    ck = np.broadcast_to(rng.standard_normal((1, 1, Hkv, d)), (B, T, Hkv, d)).copy()
    cv = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, S, H, d))
    o = ob.gqa_attention(q, ck, cv, p0).reshape(B, S, H, d)
    for s in range(S):
        for h in range(H):
            np.testing.assert_allclose(o[0, s, h], cv[0, :p0 + s + 1, h // (H // Hkv)].mean(0), atol=1e-13)


def _textbook_mha(q, k, v, p0):
    """Per-head scaled dot-product attention with an explicit lower-triangular mask."""
    B, S, H, d = q.shape
    T = k.shape[1]
    o = np.zeros((B, S, H, d))
    for b in range(B):
        for h in range(H):
            sc = q[b, :, h] @ k[b, :, h].T / math.sqrt(d)
            for s in range(S):
                e = np.exp(sc[s, :p0 + s + 1] - sc[s, :p0 + s + 1].max())
                o[b, s, h] = (e / e.sum()) @ v[b, :p0 + s + 1, h]
    return o.reshape(B, S, H * d)


def test_gqa_with_all_kv_heads_is_mha():
    rng = _rng(9)
    B, S, H, d, p0 = 2, 7, 4, 8, 3
    q = rng.standard_normal((B, S, H, d))
    ck = rng.standard_normal((B, p0 + S + 2, H, d))
    cv = rng.standard_normal((B, p0 + S + 2, H, d))
    np.testing.assert_allclose(ob.gqa_attention(q, ck, cv, p0),
                               _textbook_mha(q, ck[:, :p0 + S], cv[:, :p0 + S], p0), atol=1e-13)


def test_gqa_with_one_kv_head_is_mqa():
    """Multi-query attention: one K/V head shared by every query head (the
    LLM-Foundry MultiQueryAttention of "LLaMa-1/2/3 原理+源码", GQA section)."""
    rng = _rng(10)
    B, S, H, d, p0 = 2, 6, 8, 4, 0
    q = rng.standard_normal((B, S, H, d))
    k = rng.standard_normal((B, S, 1, d))
    v = rng.standard_normal((B, S, 1, d))
    qh = np.transpose(q, (0, 2, 1, 3))                       # [B, H, S, d]
    sc = qh @ np.transpose(k, (0, 2, 3, 1)) / math.sqrt(d)   # [B, H, S, S] (k broadcast over heads)
    sc = sc + np.triu(np.full((S, S), -np.inf), 1)
    e = np.exp(sc - sc.max(-1, keepdims=True))
    o = (e / e.sum(-1, keepdims=True)) @ np.transpose(v, (0, 2, 1, 3))
    mqa = np.transpose(o, (0, 2, 1, 3)).reshape(B, S, H * d)
    np.testing.assert_allclose(ob.gqa_attention(q, k, v, p0), mqa, atol=1e-13)


# ----------------------------------------------------------------------------- FFN
def test_silu_values():
    assert ob.silu(np.array(0.0)) == 0.0
    assert abs(ob.silu(np.array(1.0)) - 1 / (1 + math.exp(-1))) < 1e-16
    assert abs(ob.silu(np.array(40.0)) - 40.0) < 1e-12
    assert abs(ob.silu(np.array(-40.0))) < 1e-15
    # sigmoid symmetry: silu(a) - silu(-a) = a
    a = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(ob.silu(a) - ob.silu(-a), a, atol=1e-14)


def test_swiglu_ffn_on_one_hot_rows():
    """With x = e_c, w1 x = w1[:, c] and w3 x = w3[:, c]: out = w2 (silu(w1[:,c]) * w3[:,c])."""
    rng = _rng(11)
    D, F = 6, 10
    w1, w3, w2 = rng.standard_normal((F, D)), rng.standard_normal((F, D)), rng.standard_normal((D, F))
    for c in range(D):
        x = np.zeros((1, D))
        x[0, c] = 1.0
        a, b = w1[:, c], w3[:, c]
        expect = w2 @ (a / (1 + np.exp(-a)) * b)
        np.testing.assert_allclose(ob.swiglu_ffn(x, w1, w3, w2)[0], expect, atol=1e-13)


# ----------------------------------------------------------------------------- block
SMALL = dict(D=16, H=4, F=48)


def _run_block(x, w, ck, cv, p0, H, Hkv, **kw):
    return ob.block_forward(x, w, ck, cv, p0, H, Hkv, 1e-5, 1e4, **kw)


@pytest.mark.parametrize("Hkv", [1, 2, 4])
@pytest.mark.parametrize("p0", [0, 3])
def test_brute_force_matches_on_tiny_shapes(Hkv, p0):
    rng = _rng(12 + Hkv + p0)
    B, S, D, H, F = 2, 5, SMALL["D"], SMALL["H"], SMALL["F"]
    d = D // H
    w = _rand_weights(rng, D, H, Hkv, F)
    x0 = rng.standard_normal((B, p0, D))
    x = rng.standard_normal((B, S, D))
    ck, cv = _cache(B, p0 + S, Hkv, d)
    bk = [[[[0.0] * d for _ in range(Hkv)] for _ in range(p0 + S)] for _ in range(B)]
    bv = [[[[0.0] * d for _ in range(Hkv)] for _ in range(p0 + S)] for _ in range(B)]
    wl_ = {k: v.tolist() for k, v in w.items()}
    if p0:
        _run_block(x0, w, ck, cv, 0, H, Hkv)
        brute.block_forward(x0.tolist(), wl_, bk, bv, 0, H, Hkv, 1e-5, 1e4)
    got = _run_block(x, w, ck, cv, p0, H, Hkv)
    ref = np.array(brute.block_forward(x.tolist(), wl_, bk, bv, p0, H, Hkv, 1e-5, 1e4))
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(ck, np.array(bk), atol=1e-12)
    np.testing.assert_allclose(cv, np.array(bv), atol=1e-12)


def test_kv_cache_decode_equals_full_prefill():
    rng = _rng(20)
    B, D, H, Hkv, F = 2, 16, 4, 2, 48
    a, nb = 5, 4
    w = _rand_weights(rng, D, H, Hkv, F)
    x = rng.standard_normal((B, a + nb, D))
    ck, cv = _cache(B, a + nb, Hkv, D // H)
    full = _run_block(x, w, ck, cv, 0, H, Hkv)
    ck2, cv2 = _cache(B, a + nb, Hkv, D // H)
    first = _run_block(x[:, :a], w, ck2, cv2, 0, H, Hkv)
    steps = [_run_block(x[:, a + t:a + t + 1], w, ck2, cv2, a + t, H, Hkv) for t in range(nb)]
    np.testing.assert_allclose(np.concatenate([first] + steps, axis=1), full, atol=1e-12)
    np.testing.assert_allclose(ck2, ck, atol=1e-13)
    # chunked prefill (start_pos > 0 with several tokens) gives the same rows too
    ck3, cv3 = _cache(B, a + nb, Hkv, D // H)
    c1 = _run_block(x[:, :3], w, ck3, cv3, 0, H, Hkv)
    c2 = _run_block(x[:, 3:], w, ck3, cv3, 3, H, Hkv)
    np.testing.assert_allclose(np.concatenate([c1, c2], axis=1), full, atol=1e-12)


def test_row_selection_equals_full_rows():
    rng = _rng(21)
    B, S, D, H, Hkv, F = 2, 9, 16, 4, 2, 48
    w = _rand_weights(rng, D, H, Hkv, F)
    x = rng.standard_normal((B, S, D))
    ck, cv = _cache(B, S, Hkv, D // H)
    full = _run_block(x, w, ck, cv, 0, H, Hkv)
    ck2, cv2 = _cache(B, S, Hkv, D // H)
    rows = [0, 4, 8]
    part = _run_block(x, w, ck2, cv2, 0, H, Hkv, rows=rows)
    np.testing.assert_allclose(part, full[:, rows], atol=1e-13)


def test_causality_and_batch_independence():
    rng = _rng(22)
    B, S, D, H, Hkv, F = 3, 8, 16, 4, 2, 48
    w = _rand_weights(rng, D, H, Hkv, F)
    x = rng.standard_normal((B, S, D))
    ck, cv = _cache(B, S, Hkv, D // H)
    ref = _run_block(x, w, ck, cv, 0, H, Hkv)
    for t in (2, 5):
        xp = x.copy()
        xp[:, t] += rng.standard_normal((B, D))
        ck, cv = _cache(B, S, Hkv, D // H)
        got = _run_block(xp, w, ck, cv, 0, H, Hkv)
        np.testing.assert_array_equal(got[:, :t], ref[:, :t])
        assert np.all(np.abs(got[:, t] - ref[:, t]) > 0)
    ck, cv = _cache(1, S, Hkv, D // H)
    one = _run_block(x[1:2], w, ck, cv, 0, H, Hkv)
    np.testing.assert_allclose(one, ref[1:2], atol=1e-13)


def test_zero_weights_structure():
    rng = _rng(23)
    B, S, D, H, Hkv, F = 2, 5, 16, 4, 2, 48
    w = _rand_weights(rng, D, H, Hkv, F)
    x = rng.standard_normal((B, S, D))
    z = {k: (np.zeros_like(v) if k.startswith("w") else v) for k, v in w.items()}
    ck, cv = _cache(B, S, Hkv, D // H)
    np.testing.assert_array_equal(_run_block(x, z, ck, cv, 0, H, Hkv), x)
    # w2 = 0: out = h = x + attention
    w2z = dict(w, w2=np.zeros_like(w["w2"]))
    tr = {}
    ck, cv = _cache(B, S, Hkv, D // H)
    out = _run_block(x, w2z, ck, cv, 0, H, Hkv, trace=tr)
    np.testing.assert_array_equal(out, tr["h"])


def test_stack_greedy_token_lowest_index_on_ties():
    rng = _rng(24)
    B, S, D, H, Hkv, F, V = 2, 3, 16, 4, 2, 48, 11
    layers = [_rand_weights(rng, D, H, Hkv, F) for _ in range(2)]
    emb = rng.standard_normal((V, D))
    w_out = rng.standard_normal((V, D))
    w_out[7] = w_out[3]          # identical rows: equal logits at ids 3 and 7
    tok = rng.integers(0, V, (B, S))
    caches = [_cache(B, S, Hkv, D // H) for _ in layers]
    logits, nxt = ob.stack_forward(tok, emb, layers, np.ones(D), w_out, caches, 0, H, Hkv, 1e-5, 1e4)
    assert logits.shape == (B, V)
    assert np.all(logits[:, 3] == logits[:, 7])
    for b in range(B):
        assert nxt[b] == min(i for i in range(V) if logits[b, i] == logits[b].max())
    # the stack is the composition of the block, the final norm and the projection
    h = emb[tok]
    caches2 = [_cache(B, S, Hkv, D // H) for _ in layers]
    for lw, (ck, cv) in zip(layers, caches2):
        h = _run_block(h, lw, ck, cv, 0, H, Hkv)
    np.testing.assert_allclose(logits, ob.rms_norm(h[:, -1], np.ones(D), 1e-5) @ w_out.T, atol=1e-12)


# ----------------------------------------------------------------------------- planted mistakes
def _pins_pass():
    tests = [test_rmsnorm_unit_weight_rows_have_unit_rms, test_rmsnorm_printed_row_statistics,
             test_rope_pairing_matches_printed_view_as_complex_and_polar, test_rope_hand_values_d4,
             test_rope_equals_complex_multiply, test_softmax_rows_sum_to_one_and_mask,
             test_equal_keys_give_mean_of_visible_values, test_gqa_with_all_kv_heads_is_mha,
             test_gqa_with_one_kv_head_is_mqa, test_silu_values, test_swiglu_ffn_on_one_hot_rows,
             test_kv_cache_decode_equals_full_prefill, test_zero_weights_structure]
    for t in tests:
        try:
            t()
        except AssertionError:
            return False
    for Hkv in (1, 2, 4):
        for p0 in (0, 3):
            try:
                test_brute_force_matches_on_tiny_shapes(Hkv, p0)
            except AssertionError:
                return False
    return True


def _mutants():
    orig_rms, orig_freq, orig_rope = ob.rms_norm, ob.rope_inv_freq, ob.apply_rope
    orig_repeat, orig_mask, orig_silu = ob.repeat_kv, ob.causal_mask, ob.silu

    def rms_eps_outside(x, w, eps):
        x = np.asarray(x, float)
        return x / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + eps) * w

    def rms_centred(x, w, eps):
        x = np.asarray(x, float)
        xc = x - x.mean(-1, keepdims=True)
        return xc / np.sqrt(np.mean(xc * xc, -1, keepdims=True) + eps) * w

    def freq_wrong_exponent(d, theta):
        return 1.0 / (float(theta) ** (np.arange(d // 2) / d))

    def rope_half_split(u, pos, theta):
        d = u.shape[-1]
        perm = np.r_[np.arange(0, d, 2), np.arange(1, d, 2)]
        inv = np.argsort(perm)
        return orig_rope(np.asarray(u, float)[..., inv], pos, theta)[..., perm]

    def rope_wrong_sign(u, pos, theta):
        return orig_rope(u, [-p for p in pos], theta)

    def repeat_modulo(x, n_rep):
        return np.tile(x, (1, 1, n_rep, 1)) if n_rep > 1 else x

    def mask_off_by_one(S, p0):
        T = p0 + S
        return np.where(np.arange(T)[None] >= p0 + np.arange(S)[:, None], -np.inf, 0.0) if S > 1 else np.zeros((S, T))

    def silu_sigmoid_only(a):
        return 1.0 / (1.0 + np.exp(-a))

    return {
        "eps outside sqrt": ("rms_norm", rms_eps_outside),
        "mean centring": ("rms_norm", rms_centred),
        "theta exponent i/d": ("rope_inv_freq", freq_wrong_exponent),
        "half-split pairing": ("apply_rope", rope_half_split),
        "rotation sign": ("apply_rope", rope_wrong_sign),
        "kv head h % Hkv": ("repeat_kv", repeat_modulo),
        "mask hides the diagonal": ("causal_mask", mask_off_by_one),
        "silu without the a factor": ("silu", silu_sigmoid_only),
    }, dict(rms_norm=orig_rms, rope_inv_freq=orig_freq, apply_rope=orig_rope, repeat_kv=orig_repeat,
            causal_mask=orig_mask, silu=orig_silu)


def test_pins_catch_planted_mistakes():
    assert _pins_pass()
    mutants, originals = _mutants()
    for name, (attr, fn) in mutants.items():
        setattr(ob, attr, fn)
        try:
            caught = not _pins_pass()
        finally:
            setattr(ob, attr, originals[attr])
        assert caught, f"no pin caught the planted mistake: {name}"
    assert _pins_pass()
