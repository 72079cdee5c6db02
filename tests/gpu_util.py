"""Shared helpers of the GPU parity tests: device checks and the tolerance rule.

Tolerance (bf16 storage, fp32 arithmetic): relative Frobenius error <= 1e-2
and max|got - ref| / max(1, max|ref|) <= 2e-2.  fp32: both <= 1e-4.  The raw
max-abs error is reported beside them.
"""
import numpy as np
import pytest
import torch

BF16_TOL = dict(relf=1e-2, maxabs=2e-2)
F32_TOL = dict(relf=1e-4, maxabs=1e-4)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_block_amd as d
    d.lib()  # raises when the HIP library is missing: no fallback
    return torch.device("cuda:0")


def errors(got, ref):
    g = got.detach().to("cpu").to(torch.float64).numpy() if isinstance(got, torch.Tensor) else np.asarray(got, float)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite values in the GPU result"
    diff = np.abs(g - r)
    nref = np.linalg.norm(r)
    relf = np.linalg.norm(g - r) / (nref if nref > 0 else 1.0)
    raw = float(diff.max()) if diff.size else 0.0
    norm_max = raw / max(1.0, float(np.abs(r).max()) if r.size else 1.0)
    return dict(relf=float(relf), maxabs=norm_max, raw_maxabs=raw)


def check(got, ref, dtype, what=""):
    tol = BF16_TOL if dtype in ("bf16", torch.bfloat16) else F32_TOL
    e = errors(got, ref)
    print(f"[parity] {what}: relF={e['relf']:.3e} maxabs/max(1,|ref|)={e['maxabs']:.3e} raw={e['raw_maxabs']:.3e}",
          flush=True)
    assert e["relf"] <= tol["relf"], (what, e)
    assert e["maxabs"] <= tol["maxabs"], (what, e)
    return e


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()
