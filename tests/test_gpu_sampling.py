"""Parity of the device next-token selection (llama_sample_top_p) with the oracle (GPU).

The kernel computes each token's weight in fp32 and its sums in fp64; the
oracle is float64 throughout.  Where the draw is unique up to that arithmetic
(boundaries far from top_p and from u) the tokens must be equal.  With a
128256-token vocabulary and a flat distribution neighbouring boundaries of the
cumulative distribution lie ~1e-5 apart, so there the test checks what is
unique -- that the device's token is kept and that u falls in its interval of
the oracle's renormalised cumulative distribution, both to within TOL -- and
that the device result is deterministic.
"""
import numpy as np
import pytest
import torch

import decoder_block_amd as dba
from oracle import sample as osm
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-5   # probability units; fp32 weights + per-thread fp32 partial sums err by ~1e-6


def _run(logits, temperature, top_p, uniforms):
    rows, vocab = logits.shape
    lg = torch.as_tensor(logits, dtype=torch.float32).cuda()
    nx = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    un = torch.as_tensor(uniforms, dtype=torch.float32).cuda()
    dba.llama_sample_top_p(lg, nx, rows, vocab, temperature, top_p, un)
    torch.cuda.synchronize()
    return nx.cpu().numpy().astype(np.int64)


def _valid(logits_row, temperature, top_p, u, tok):
    """The device token is kept and u lies in its cdf interval, both within TOL (oracle arithmetic)."""
    probs = osm.softmax_temperature(logits_row, temperature)
    order = osm.sorted_order(probs)
    ps = probs[order]
    before = np.cumsum(ps) - ps
    pos = int(np.flatnonzero(order == tok)[0])
    if before[pos] > top_p + TOL:
        return False
    s = ps[before <= top_p].sum()
    lo, hi = before[pos] / s, (before[pos] + ps[pos]) / s
    return lo - TOL <= u <= hi + TOL


def test_hand_computed_cases_exact():
    need_gpu()
    print("case sample hand-computed", flush=True)
    row = np.log(np.array([0.15, 0.5, 0.05, 0.3]))
    cases = [(0.79, 0.0, 1), (0.79, 0.62, 1), (0.79, 0.63, 3), (0.79, 0.999, 3), (0.81, 0.52, 1), (0.81, 0.53, 3),
             (0.81, 0.842, 3), (0.81, 0.8422, 0), (0.81, 0.99, 0), (0.0, 0.9, 1), (1.0, 0.97, 2)]
    for top_p, u, want in cases:
        got = _run(row[None, :], 1.0, top_p, [u])[0]
        assert got == want == osm.sample_row(row, 1.0, top_p, u), (top_p, u, got, want)


def test_small_vocab_exact_where_unambiguous():
    need_gpu()
    print("case sample small vocab", flush=True)
    rng = np.random.default_rng(21)
    rows, vocab = 256, 97
    lg = rng.normal(0.0, 3.0, (rows, vocab)).astype(np.float32)
    for T, p in ((1.0, 0.9), (0.7, 0.5), (1.3, 1.0), (2.0, 0.99)):
        u = rng.random(rows).astype(np.float32)
        got = _run(lg, T, p, u)
        want = osm.sample(lg, T, p, u)
        for r in range(rows):
            if got[r] != want[r]:
                mp, mu = osm.decision_margins(lg[r], T, p, float(u[r]))
                assert min(mp, mu) < TOL, (T, p, r, got[r], want[r], mp, mu)
        assert np.mean(got == want) > 0.98


@pytest.mark.parametrize("T,p", [(0.8, 0.95), (1.0, 0.5), (1.5, 1.0), (0.6, 0.99)])
def test_full_vocab_valid_and_deterministic(T, p):
    need_gpu()
    print(f"case sample 64 x 128256 T={T} p={p}", flush=True)
    rng = np.random.default_rng(int(T * 100 + p * 1000))
    rows, vocab = 64, 128256
    lg = rng.normal(0.0, 1.3, (rows, vocab)).astype(np.float32)
    lg[:, 777] += 6.0                                     # one strong token in every row
    u = rng.random(rows).astype(np.float32)
    got = _run(lg, T, p, u)
    again = _run(lg, T, p, u)
    np.testing.assert_array_equal(got, again)
    for r in range(rows):
        assert _valid(lg[r], T, p, float(u[r]), int(got[r])), (r, got[r])
    want = osm.sample(lg, T, p, u)
    print(f"  exact matches {np.mean(got == want):.2f}", flush=True)


def test_greedy_and_tiny_nucleus_and_ties():
    need_gpu()
    print("case sample greedy / tiny nucleus / ties", flush=True)
    rng = np.random.default_rng(5)
    rows, vocab = 8, 5000
    lg = rng.normal(0.0, 1.0, (rows, vocab)).astype(np.float32)
    lg[3, [100, 4000]] = 50.0                             # exact tie at the top: the lower id wins
    am = osm.sample(lg, 0.0, 0.9, np.zeros(rows))
    assert am[3] == 100
    np.testing.assert_array_equal(_run(lg, 0.0, 0.9, np.zeros(rows)), am)
    u = rng.random(rows)
    np.testing.assert_array_equal(_run(lg, 0.8, 1e-7, u), am)   # only the most probable token is kept
    # the tie split by u: kept {100, 4000} for a nucleus just above one token's mass
    p3 = osm.softmax_temperature(lg[3], 1.0)
    top = float(p3[100]) * 1.0001
    row3 = lg[3:4]
    assert _run(row3, 1.0, top, [0.25])[0] == 100
    assert _run(row3, 1.0, top, [0.75])[0] == 4000


def test_equal_logits_many_ties():
    """All logits equal: every token has the same probability, ordered by id; the
    cut keeps floor(top_p * V) + 1 tokens and u picks floor(u * kept) (the tie
    resolution's binary search over ids)."""
    need_gpu()
    print("case sample equal logits", flush=True)
    V = 1000
    lg = np.full((4, V), 0.25, dtype=np.float32)
    u = np.array([0.0, 0.3, 0.77, 0.999], dtype=np.float32).astype(np.float64)   # the values the device sees
    # top_p * V kept well away from an integer: the cut is then the same in fp32 and fp64
    for p in (0.4567, 0.0013, 0.9123):
        kept = int(np.floor(p * V)) + 1
        got = _run(lg, 1.0, p, u)
        np.testing.assert_array_equal(got, np.floor(u * kept).astype(np.int64))
        np.testing.assert_array_equal(got, osm.sample(lg, 1.0, p, u))
    np.testing.assert_array_equal(_run(lg, 1.0, 1.0, u), np.floor(u * V).astype(np.int64))


def test_equal_logits_full_vocab_fallback():
    """128256 equal logits: every token stays in the search range, more than the
    candidate list holds, so the selection keeps reading the row; the result is
    still the closed form floor(u * kept)."""
    need_gpu()
    print("case sample equal logits, 128256 tokens", flush=True)
    V = 128256
    lg = np.full((2, V), -1.5, dtype=np.float32)
    u = np.array([0.1234, 0.87], dtype=np.float32).astype(np.float64)
    p = 0.61234                                         # p * V = 78536.4...
    kept = int(np.floor(p * V)) + 1
    np.testing.assert_array_equal(_run(lg, 1.0, p, u), np.floor(u * kept).astype(np.int64))
