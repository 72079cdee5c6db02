"""Pure-Python loop version of the decoder block for tiny shapes (test infrastructure only).

Written independently of ``oracle.block``: nested lists, Python ``complex``
for the rotary multiply, an explicit -inf mask, an explicit copy of every kv
head n_rep times (repeat_kv), and ``math.exp`` for the softmax.  Used only to
cross-check ``oracle.block`` on shapes of a few dozen elements.
Layouts: x[b][s][c]; weights W[out][in]; cache[b][t][kv_head][e].
"""
from __future__ import annotations

import math
from typing import List


def _matvec(W, v):
    return [sum(W[o][i] * v[i] for i in range(len(v))) for o in range(len(W))]


def rms_norm_row(v, g, eps):
    ms = sum(a * a for a in v) / len(v)
    r = 1.0 / math.sqrt(ms + eps)
    return [a * r * gi for a, gi in zip(v, g)]


def rope_vec(u, pos, theta):
    """u viewed as complex numbers u[2i] + 1j*u[2i+1], each times e^{1j*pos*theta^(-2i/d)}."""
    d = len(u)
    out = []
    for i in range(d // 2):
        w = theta ** (-(2.0 * i) / d)
        z = complex(u[2 * i], u[2 * i + 1]) * complex(math.cos(pos * w), math.sin(pos * w))
        out += [z.real, z.imag]
    return out


def block_forward(x, w, cache_k, cache_v, start_pos, n_heads, n_kv_heads, eps, theta) -> List:
    B, S, D = len(x), len(x[0]), len(x[0][0])
    d = D // n_heads
    n_rep = n_heads // n_kv_heads
    out = [[None] * S for _ in range(B)]
    # projections, RoPE and the cache write for every new position
    qs = [[None] * S for _ in range(B)]
    for b in range(B):
        for s in range(S):
            xn = rms_norm_row(x[b][s], w["attention_norm"], eps)
            q = _matvec(w["wq"], xn)
            k = _matvec(w["wk"], xn)
            v = _matvec(w["wv"], xn)
            p = start_pos + s
            qs[b][s] = [rope_vec(q[h * d:(h + 1) * d], p, theta) for h in range(n_heads)]
            for j in range(n_kv_heads):
                cache_k[b][p][j] = rope_vec(k[j * d:(j + 1) * d], p, theta)
                cache_v[b][p][j] = list(v[j * d:(j + 1) * d])
    T = start_pos + S
    for b in range(B):
        # explicit repeat_kv: a full copy of every kv head for each of its n_rep q heads
        keys = [[list(cache_k[b][t][hq // n_rep]) for hq in range(n_heads)] for t in range(T)]
        vals = [[list(cache_v[b][t][hq // n_rep]) for hq in range(n_heads)] for t in range(T)]
        for s in range(S):
            o = []
            for hq in range(n_heads):
                q = qs[b][s][hq]
                sc = []
                for t in range(T):
                    val = sum(q[e] * keys[t][hq][e] for e in range(d)) / math.sqrt(d)
                    if S > 1 and t > start_pos + s:
                        val = -math.inf
                    sc.append(val)
                m = max(sc)
                ex = [0.0 if z == -math.inf else math.exp(z - m) for z in sc]
                tot = sum(ex)
                o += [sum(ex[t] / tot * vals[t][hq][e] for t in range(T)) for e in range(d)]
            h = [a + c for a, c in zip(x[b][s], _matvec(w["wo"], o))]
            hn = rms_norm_row(h, w["ffn_norm"], eps)
            a1 = _matvec(w["w1"], hn)
            a3 = _matvec(w["w3"], hn)
            g = [(u / (1.0 + math.exp(-u))) * z for u, z in zip(a1, a3)]
            out[b][s] = [a + c for a, c in zip(h, _matvec(w["w2"], g))]
    return out
