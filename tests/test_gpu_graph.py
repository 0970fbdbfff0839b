"""The entry points under HIP graph capture: a graph holding a prefill, a GQA
decode and an MLA decode is replayed several times, with unrelated eager work
and synchronisation between replays; every replay must reproduce the eager
results bit for bit (the launches record no memset nodes)."""
import pytest
import torch

import workloads
from parity import dev_bf16

pytestmark = pytest.mark.gpu


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def test_graph_replays_match_eager(gpu):
    wp = workloads.gen_prefill(1, 8, 2, 300, 128, dtype="bf16", seed=31)
    wd = workloads.gen_decode_gqa(2, 32, 8, 1000, kv_cap=1024, seed=32)
    wm = workloads.gen_decode_mla(1, 128, 700, kv_cap=704, seed=33)
    pq, pk, pv = dev_bf16(wp.q), dev_bf16(wp.k), dev_bf16(wp.v)
    dq, dk, dv = dev_bf16(wd.q), dev_bf16(wd.k), dev_bf16(wd.v)
    mq, mc = dev_bf16(wm.q), dev_bf16(wm.ckv)

    ref = [gpu.attn_prefill_causal(pq, pk, pv, wp.scale),
           gpu.attn_decode_gqa(dq, dk, dv, wd.kv_len, wd.scale),
           gpu.attn_decode_mla_absorbed(mq, mc, wm.kv_len, wm.Dv, wm.scale)]
    torch.cuda.synchronize()

    outs = [(torch.empty_like(r[0]), torch.empty_like(r[1])) for r in ref]
    ws_d = torch.empty(gpu.attn_decode_gqa_workspace_bytes(2, 32, 8, wd.kv_len), dtype=torch.uint8,
                       device="cuda")
    ws_m = torch.empty(gpu.attn_decode_mla_workspace_bytes(1, 128, wm.kv_len), dtype=torch.uint8,
                       device="cuda")

    def calls():
        gpu.attn_prefill_causal(pq, pk, pv, wp.scale, out=outs[0][0], lse=outs[0][1])
        gpu.attn_decode_gqa(dq, dk, dv, wd.kv_len, wd.scale, out=outs[1][0], lse=outs[1][1], ws=ws_d)
        gpu.attn_decode_mla_absorbed(mq, mc, wm.kv_len, wm.Dv, wm.scale, out=outs[2][0],
                                     lse=outs[2][1], ws=ws_m)

    calls()  # eager warm-up with the graph's own buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()

    other = workloads.gen_decode_gqa(1, 8, 2, 333, seed=34)
    oq, ok, ov = dev_bf16(other.q), dev_bf16(other.k), dev_bf16(other.v)
    for rep in range(4):
        for o, l in outs:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(outs, ref):
            assert _same(o, ro) and _same(l, rl), "replay %d differs from eager" % rep
        # unrelated eager work (reuses the default-stream workspace) between replays
        gpu.attn_decode_gqa(oq, ok, ov, other.kv_len, other.scale)
        torch.cuda.synchronize()
