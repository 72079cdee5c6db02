"""The allocation-free decode attention entry point (GPU).

llama_gqa_attn_decode_static runs the same kernels as llama_gqa_attn_decode with
the split-K partials in the library's static per-GPU scratch array instead of a
caller workspace.  Through the C ABI, two calls in a row (the second with a
smaller batch and shorter context, over the first call's leftovers in the
scratch) must give exactly the outputs and appended cache rows of the
workspace entry point on the same inputs, and follow the oracle.  (A call whose
partials exceed the scratch is refused on the host: tests/test_abi_host.py.)"""
import ctypes

import numpy as np
import pytest
import torch

import decoder_block_amd as dba
import workloads as wl
from oracle import block as ob
from tests.gpu_util import check, f64, need_gpu

pytestmark = pytest.mark.gpu


def _case(B, p0, H, Hkv, d, tid):
    dev = torch.device("cuda:0")
    args = dba.ModelArgs(dim=H * d, n_heads=H, n_kv_heads=Hkv, multiple_of=256, max_batch_size=B,
                         max_seq_len=p0 + 2)
    q, k, v = (wl.normal(s, 1.0, "bf16", 0, 0, tid + i) for i, s in
               enumerate(((B, 1, H, d), (B, 1, Hkv, d), (B, 1, Hkv, d))))
    ck = torch.zeros(B, p0 + 2, Hkv, d, dtype=torch.bfloat16)
    ck[:, :p0] = wl.normal((B, p0, Hkv, d), 1.0, "bf16", 0, 0, tid + 3)
    cv = torch.zeros_like(ck)
    cv[:, :p0] = wl.normal((B, p0, Hkv, d), 1.0, "bf16", 0, 0, tid + 4)
    return args, [t.to(dev) for t in (q, k, v)], ck, cv


@pytest.mark.parametrize("first,second", [
    ((1, 8300, 32, 8, 128), (1, 3000, 32, 8, 128)),     # many splits, then fewer over the leftovers
    ((8, 2000, 16, 2, 128), (2, 300, 8, 2, 64)),        # another head_dim and head count second
])
def test_static_scratch_decode_matches_workspace_call(first, second):
    dev = need_gpu()
    lib = dba.lib()
    assert dba.llama_static_scratch_bytes() == 8 << 20
    for n, (B, p0, H, Hkv, d) in enumerate((first, second)):
        print(f"case static-scratch decode call {n}: B={B} p0={p0} H={H} Hkv={Hkv} d={d}", flush=True)
        args, (q, k, v), ck, cv = _case(B, p0, H, Hkv, d, 500 + 10 * n)
        need = dba.llama_attn_decode_workspace_size(args, B, p0)
        assert 0 < need <= dba.llama_static_scratch_bytes()
        ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=dev)
        ck_a, cv_a = ck.to(dev), cv.to(dev)
        ck_b, cv_b = ck.to(dev), cv.to(dev)
        out_a = torch.empty(B, 1, H * d, dtype=torch.bfloat16, device=dev)
        out_b = torch.full_like(out_a, float("nan"))
        st = torch.cuda.current_stream().cuda_stream
        ca = ctypes.byref(args.c())
        assert lib.llama_gqa_attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), ck_a.data_ptr(), cv_a.data_ptr(),
                                         out_a.data_ptr(), ca, B, p0, ws.data_ptr(), need, dba.LLAMA_BF16, st) == 0
        assert lib.llama_gqa_attn_decode_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), ck_b.data_ptr(),
                                                cv_b.data_ptr(), out_b.data_ptr(), ca, B, p0, dba.LLAMA_BF16,
                                                st) == 0
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), "static-scratch output differs from the workspace call"
        assert torch.equal(ck_a, ck_b) and torch.equal(cv_a, cv_b)
        rck, rcv = f64(ck), f64(cv)
        rck[:, p0] = f64(k)[:, 0]
        rcv[:, p0] = f64(v)[:, 0]
        check(out_b, ob.gqa_attention(f64(q), rck, rcv, p0), "bf16", f"static-scratch decode call {n}")
