"""attn_decode_gqa_noalloc (the GQA decode that allocates nothing and keeps
its split partials in the library's static scratch) against attn_decode_gqa
with a caller workspace, called through the C ABI: two calls in a row, the
second smaller, each bit for bit equal to the workspace form and within the
comparison rule of the fp64 oracle; a shape whose partials exceed the
scratch is refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_bf16, dev_bf16, host

pytestmark = pytest.mark.gpu

WS = 4  # ATTN_ERR_WORKSPACE


def _noalloc_cabi(lib, q, k, v, o, lse, kv_len, scale):
    B, Hq, D = q.shape
    _, Hkv, kv_cap, _ = k.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.attn_decode_gqa_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), B, Hq, Hkv, kv_len, kv_cap, D, scale, stream)


def test_noalloc_equals_workspace_form_twice_then_refuses_too_big(gpu):
    lib = gpu.load()
    cases = [workloads.make("decode_gqa_llama3_8b_4k"),                       # 0.5 MiB of partials
             workloads.gen_decode_gqa(2, 16, 4, 1000, D=128, kv_cap=1024, seed=8)]  # smaller
    for w in cases:
        q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
        o = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
        st = _noalloc_cabi(lib, q, k, v, o, lse, w.kv_len, w.scale)
        assert st == 0, gpu.last_error()
        o_ws, l_ws = gpu.attn_decode_gqa(q, k, v, w.kv_len, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ws.view(torch.int16))
        assert torch.equal(lse, l_ws)
        o_ref, l_ref = oracle.decode_gqa(w.q, w.k, w.v, w.kv_len, w.scale)
        check_bf16(host(o), o_ref, host(lse), l_ref, "noalloc %s" % ((w.B, w.Hq, w.Hkv, w.kv_len),))
    # 31 sequences x 8 K/V heads of group 16 split in two: 4.2 MB of partials
    B, Hq, Hkv, L = 31, 128, 8, 512
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, L, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full((B, Hq, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq), 7.0, dtype=torch.float32, device="cuda")
    assert _noalloc_cabi(lib, q, k, k, o, lse, L, 0.125) == WS
    assert "static scratch" in gpu.last_error()
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
