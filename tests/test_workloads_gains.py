"""The seeded RMSNorm weights of the test workloads are strong enough to catch a
gain mistake: on the oracle (CPU), swapping attention_norm and ffn_norm, or
dropping either weight, moves the block output far outside the bf16 parity
tolerance (relative Frobenius 1e-2), so a GPU path with such a mistake cannot
pass the parity tests that use these weights.

The shape is that of the dim-2048 test workloads (16 query heads over 8 kv
heads), which carry the GPU tests of every fused normalisation path.  With
weights N(0, 0.02) the attention and FFN branches grow with dim (at dim 2048 they
are about half the output's norm, at dim 512 an eighth), and a gain mistake moves
the output in proportion: at dim 512 dropping a 1 + N(0, 0.2^2) weight moves it
only about 2 %."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import block as ob


def _relf(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("gains", ["normal", "pow2"])
def test_gain_mistakes_leave_the_tolerance(gains):
    w = wl.Workload(40, "gain-check", "bf16", 2048, 16, 8, 1536, 256, 0.25, 1e-5, 5e5, batch=2, prefill_len=24,
                    decode_steps=0, norm_gains=gains)
    assert wl.block_weights(w)["w1"].shape == (1536, 2048)
    wts = {k: v.to(torch.float64).numpy() for k, v in wl.block_weights(w).items()}
    assert not np.allclose(wts["attention_norm"], 1.0) and not np.allclose(wts["ffn_norm"], 1.0)
    assert not np.allclose(wts["attention_norm"], wts["ffn_norm"])
    if gains == "pow2":
        assert set(np.unique(wts["ffn_norm"])) <= {0.5, 1.0, 2.0}
    x = wl.activations(w).to(torch.float64).numpy()
    shape = (w.batch, w.max_seq_len, w.n_kv_heads, w.head_dim)

    def run(wv):
        ck, cv = np.zeros(shape), np.zeros(shape)
        return ob.block_forward(x, wv, ck, cv, 0, w.n_heads, w.n_kv_heads, w.norm_eps, w.rope_theta)

    ref = run(wts)
    one = np.ones(w.dim)
    mistakes = {
        "swapped norms": dict(wts, attention_norm=wts["ffn_norm"], ffn_norm=wts["attention_norm"]),
        "attention_norm dropped": dict(wts, attention_norm=one),
        "ffn_norm dropped": dict(wts, ffn_norm=one),
    }
    for name, wv in mistakes.items():
        assert _relf(run(wv), ref) > 5e-2, name


def test_gain_tensors_differ_per_layer_and_norm():
    w = wl.WORKLOADS[5].scaled(norm_gains="pow2", dim=64, n_heads=4, n_kv_heads=2)
    a, b = wl.block_weights(w, 0), wl.block_weights(w, 1)
    assert not torch.equal(a["attention_norm"], b["attention_norm"])
    assert not torch.equal(a["attention_norm"], a["ffn_norm"])
    unit = wl.block_weights(wl.WORKLOADS[1])
    assert torch.all(unit["attention_norm"] == 1) and torch.all(unit["ffn_norm"] == 1)
