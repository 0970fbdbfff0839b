"""Serving shapes on the GPU (through the C ABI) against the fp64 oracle:
chunked prefill against a K/V cache (the bottom-right causal mask of
第11节 §3) and decode batches whose sequences have their own lengths, with
the lengths in device memory so one captured graph serves new lengths."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_bf16, dev_bf16, host

pytestmark = pytest.mark.gpu


def _lens(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device="cuda")


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


# ------------------------------------------------------------- chunked prefill ---
def _chunked(gpu, w, lens=None):
    o, lse = gpu.attn_prefill_chunked(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                      _lens(w.kv_lens if lens is None else lens), w.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("B,Hq,Hkv,Nq,lens,kv_cap", [
    (1, 4, 1, 1, [1], 1),                      # one token, nothing cached
    (1, 4, 2, 1, [777], 800),                  # a decode step through the prefill kernel
    (2, 8, 2, 64, [64, 200], 256),             # no history / a partial history tile
    (2, 8, 2, 100, [100, 613], 640),           # ragged chunk, partial last key tile
    (1, 32, 8, 300, [1300], 1400),             # two query tiles, the second partial
    (3, 16, 4, 257, [257, 1000, 2048], 2048),  # mixed history lengths in one batch
    (1, 4, 4, 513, [4000], 4096),              # history not a multiple of the key tile
    (2, 2, 1, 256, [256, 4096], 4100),         # whole query tile, long history
    (1, 8, 2, 16, [6000], 6000),               # a short chunk: keys split over 8 workgroups
    (2, 4, 1, 100, [7000, 150], 7000)])        # split ranges that end before the chunk
def test_prefill_chunked_matches_oracle(gpu, B, Hq, Hkv, Nq, lens, kv_cap):
    """Slots past each sequence's length hold NaN: a kernel that read them
    would fail the finiteness check."""
    w = workloads.gen_prefill_chunked(B, Hq, Hkv, Nq, lens, D=128, kv_cap=kv_cap, seed=Nq + Hq)
    o, lse = _chunked(gpu, w)
    o_ref, lse_ref = oracle.prefill_chunked(w.q, w.k, w.v, w.kv_lens, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "chunked %s" % ((B, Hq, Hkv, Nq, lens),))


def test_prefill_chunked_without_history_is_causal_prefill(gpu):
    """A chunk that is the whole sequence (kv_len = Nq = kv_cap) is the causal
    prefill, bit for bit (the same kernel code with no history offset)."""
    w = workloads.gen_prefill(2, 8, 2, 700, 128, dtype="bf16", seed=41)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    o_c, l_c = gpu.attn_prefill_chunked(q, k, v, _lens([700, 700]), w.scale)
    o_p, l_p = gpu.attn_prefill_causal(q, k, v, w.scale)
    torch.cuda.synchronize()
    assert _same(o_c, o_p) and _same(l_c, l_p)


def test_prefill_chunked_clamps_lengths(gpu):
    """Lengths below Nq act as Nq and lengths above kv_cap as kv_cap (the
    kernel never reads outside the first kv_cap slots)."""
    w = workloads.gen_prefill_chunked(2, 8, 2, 70, [300, 300], kv_cap=300, seed=42)
    o, lse = _chunked(gpu, w, lens=[5, 10 ** 6])
    o_ref, lse_ref = oracle.prefill_chunked(w.q, w.k, w.v, [70, 300], w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "chunked clamp")


def test_prefill_chunked_4k_on_32k_workload_sampled_rows(gpu):
    """The full serving shape (a 4096-token chunk after 28672 cached tokens,
    32/8 heads): every output finite; the oracle checks the first, last and
    tile-boundary rows of every head."""
    w = workloads.make("prefill_chunked_4k_on_32k")
    o, lse = _chunked(gpu, w)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    rows = [0, 1, 63, 64, 255, 256, 2047, 4094, 4095]
    o_ref, lse_ref = oracle.prefill_chunked(w.q, w.k, w.v, w.kv_lens, w.scale, rows=rows)
    check_bf16(host(o[:, :, rows]), o_ref, host(lse[:, :, rows]), lse_ref,
               "prefill_chunked_4k_on_32k")


def test_prefill_chunked_512_on_32k_workload_sampled_rows(gpu):
    """The short-chunk serving shape (a 512-token chunk after 32256 cached
    tokens, 32/8 heads), which the launcher runs as key splits merged
    through their log-sum-exp: every output finite; the oracle checks the
    first, last and tile-boundary rows of every head."""
    w = workloads.make("prefill_chunked_512_on_32k")
    o, lse = _chunked(gpu, w)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    rows = [0, 1, 31, 32, 63, 64, 255, 256, 510, 511]
    o_ref, lse_ref = oracle.prefill_chunked(w.q, w.k, w.v, w.kv_lens, w.scale, rows=rows)
    check_bf16(host(o[:, :, rows]), o_ref, host(lse[:, :, rows]), lse_ref,
               "prefill_chunked_512_on_32k")


# ------------------------------------------------------------------ ragged GQA ---
def _check_ragged(o, lse, o_ref, lse_ref, lens, what):
    """Empty sequences: O = 0 and LSE = −∞ exactly; the rest by the rule."""
    lens = np.asarray(lens)
    empty, full = np.flatnonzero(lens == 0), np.flatnonzero(lens > 0)
    o, lse = host(o), host(lse)
    if empty.size:
        assert np.all(o[empty] == 0.0) and np.all(lse[empty] == -np.inf), what
    if full.size:
        check_bf16(o[full], o_ref[full], lse[full], lse_ref[full], what)


@pytest.mark.parametrize("Hq,Hkv,lens,max_len,kv_cap", [
    (8, 2, [0, 1, 5, 300], 300, 320),
    (32, 8, [4096, 17, 1000, 2048, 0, 3, 4095, 128], 4096, 4096),
    (4, 1, [10, 20], 1000, 1000),                  # max_kv_len only a bound
    (16, 1, [255, 256, 257, 64, 65, 63], 257, 260),
    (24, 8, [1, 1, 1], 1, 8),                       # a single split
    # 256 (b, K/V head) groups: the plan is 3 pieces of at most 768 keys,
    # lengths on and around the piece boundaries
    (8, 8, [0, 1, 767, 768, 769, 1535, 1536, 1537, 2000, 483, 1352, 184, 428, 635, 619, 1818,
            1599, 1831, 1992, 157, 284, 1736, 157, 332, 361, 1828, 719, 527, 339, 917, 1178,
            1601], 2000, 2048)])
def test_decode_gqa_ragged_matches_oracle(gpu, Hq, Hkv, lens, max_len, kv_cap):
    B = len(lens)
    w = workloads.gen_decode_gqa(B, Hq, Hkv, D=128, kv_cap=kv_cap, kv_lens=lens, seed=B + Hq)
    o, lse = gpu.attn_decode_gqa_ragged(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), _lens(lens),
                                        max_len, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_gqa_ragged(w.q, w.k, w.v, w.kv_lens, w.scale)
    _check_ragged(o, lse, o_ref, lse_ref, lens, "gqa ragged %s" % (lens,))


def test_decode_gqa_ragged_equal_lengths_is_uniform_decode(gpu):
    w = workloads.gen_decode_gqa(4, 32, 8, 1500, kv_cap=1600, seed=43)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    a = gpu.attn_decode_gqa_ragged(q, k, v, _lens([1500] * 4), 1500, w.scale)
    b = gpu.attn_decode_gqa(q, k, v, 1500, w.scale)
    torch.cuda.synchronize()
    assert _same(a[0], b[0]) and _same(a[1], b[1])


def test_decode_gqa_ragged_8k_workload(gpu):
    """32 sequences of 128..8192 keys (seeded), Llama-3-8B heads: every row
    against the oracle."""
    w = workloads.make("decode_gqa_ragged_8k")
    o, lse = gpu.attn_decode_gqa_ragged(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                        _lens(w.kv_lens), w.kv_len, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_gqa_ragged(w.q, w.k, w.v, w.kv_lens, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "decode_gqa_ragged_8k")


# ------------------------------------------------------------------ ragged MLA ---
@pytest.mark.parametrize("Hq,lens,max_len,kv_cap", [
    (16, [0, 1, 100, 512, 513, 2000], 2000, 2000),   # short rows take the residual product
    (128, [3, 40, 600], 600, 640),
    (32, [0, 200, 512], 512, 520),                   # every row short
    (144, [70, 1], 100, 100),
    (16, [int(x) for x in workloads.ragged_lengths(70, 0, 700, 7)], 700, 700)])  # > 64 sequences
def test_decode_mla_ragged_matches_oracle(gpu, Hq, lens, max_len, kv_cap):
    B = len(lens)
    w = workloads.gen_decode_mla(B, Hq, kv_cap=kv_cap, kv_lens=lens, seed=B + Hq)
    o, lse = gpu.attn_decode_mla_ragged(dev_bf16(w.q), dev_bf16(w.ckv), _lens(lens), max_len,
                                        w.Dv, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_mla_ragged(w.q, w.ckv, w.kv_lens, w.Dv, w.scale)
    _check_ragged(o, lse, o_ref, lse_ref, lens, "mla ragged %s" % (lens,))


@pytest.mark.parametrize("kv_len", [400, 3000])
def test_decode_mla_ragged_equal_lengths(gpu, kv_len):
    """Equal lengths through the ragged entry point (balanced split over the
    batch's tiles) and the uniform one (per-sequence split) both meet the
    bar against the oracle."""
    w = workloads.gen_decode_mla(2, 128, kv_len, kv_cap=kv_len, seed=44)
    q, c = dev_bf16(w.q), dev_bf16(w.ckv)
    a = gpu.attn_decode_mla_ragged(q, c, _lens([kv_len] * 2), kv_len, w.Dv, w.scale)
    b = gpu.attn_decode_mla_absorbed(q, c, kv_len, w.Dv, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q, w.ckv, kv_len, w.Dv, w.scale)
    check_bf16(host(a[0]), o_ref, host(a[1]), lse_ref, "mla ragged equal lengths")
    check_bf16(host(b[0]), o_ref, host(b[1]), lse_ref, "mla uniform")


def test_decode_mla_ragged_32k_workload_sampled_heads(gpu):
    """16 sequences of 1024..32768 latent rows: all outputs finite; the
    oracle checks 16 of the 128 heads of every sequence."""
    w = workloads.make("decode_mla_ragged_32k")
    o, lse = gpu.attn_decode_mla_ragged(dev_bf16(w.q), dev_bf16(w.ckv), _lens(w.kv_lens),
                                        w.kv_len, w.Dv, w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    hs = list(range(0, 128, 8))
    o_ref, lse_ref = oracle.decode_mla_ragged(w.q[:, hs], w.ckv, w.kv_lens, w.Dv, w.scale)
    check_bf16(host(o[:, hs]), o_ref, host(lse[:, hs]), lse_ref, "decode_mla_ragged_32k")


# ------------------------------------------------------- ragged MLA, E4M3 cache ---
def _dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


@pytest.mark.parametrize("Hq,lens,max_len,kv_cap", [
    (16, [0, 1, 100, 512, 513, 2000], 2000, 2000),   # short rows take the residual product
    (128, [3, 40, 600], 600, 640),
    (32, [0, 200, 512], 512, 520),                   # every row short
    (144, [70, 1], 100, 100),                        # a partial head group
    (16, [int(x) for x in workloads.ragged_lengths(70, 0, 700, 7)], 700, 700)])  # > 64 sequences
def test_decode_mla_ragged_fp8_matches_oracle(gpu, Hq, lens, max_len, kv_cap):
    """Ragged batch over an E4M3 latent cache (balanced rows S·c, the NaN
    code past each length): the oracle reads the same codes."""
    B = len(lens)
    w = workloads.gen_decode_mla(B, Hq, kv_cap=kv_cap, kv_lens=lens, seed=3 * B + Hq,
                                 cache_dtype="fp8")
    o, lse = gpu.attn_decode_mla_ragged_fp8(dev_bf16(w.q), _dev_u8(w.ckv), _lens(lens), max_len,
                                            w.Dv, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_mla_ragged(w.q, w.ckv, w.kv_lens, w.Dv, w.scale)
    _check_ragged(o, lse, o_ref, lse_ref, lens, "mla ragged fp8 %s" % (lens,))


def test_decode_mla_ragged_fp8_equals_bf16_copy(gpu):
    """The E4M3 ragged decode gives the same bits as the bf16 ragged decode
    over a bf16 copy of the cached values (every E4M3 value is a bf16 value,
    and both feed the same operands to the same products in the same
    order), for a batch that mixes empty, short and long sequences."""
    lens = [0, 7, 300, 513, 2500, 4096, 1]
    w = workloads.gen_decode_mla(len(lens), 128, kv_cap=4096, kv_lens=lens, seed=71,
                                 cache_dtype="fp8")
    q, kl = dev_bf16(w.q), _lens(lens)
    o8, l8 = gpu.attn_decode_mla_ragged_fp8(q, _dev_u8(w.ckv), kl, 4096, w.Dv, w.scale)
    c16 = _dev_u8(w.ckv).view(torch.float8_e4m3fn).to(torch.bfloat16)
    o16, l16 = gpu.attn_decode_mla_ragged(q, c16, kl, 4096, w.Dv, w.scale)
    torch.cuda.synchronize()
    assert _same(o8, o16) and _same(l8, l16)


def test_decode_mla_ragged_fp8_32k_workload_sampled_heads(gpu):
    """The E4M3 ragged batch as timed (16 sequences of 1024..32768 latent
    rows): all outputs finite; the oracle, reading the same codes, checks 8
    of the 128 heads of every sequence, one in each 16-head block."""
    w = workloads.make("decode_mla_ragged_fp8_32k")
    o, lse = gpu.attn_decode_mla_ragged_fp8(dev_bf16(w.q), _dev_u8(w.ckv), _lens(w.kv_lens),
                                            w.kv_len, w.Dv, w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    hs = list(range(3, 128, 16))
    o_ref, lse_ref = oracle.decode_mla_ragged(w.q[:, hs], w.ckv, w.kv_lens, w.Dv, w.scale)
    check_bf16(host(o[:, hs]), o_ref, host(lse[:, hs]), lse_ref, "decode_mla_ragged_fp8_32k")


# ------------------------------------------------------- one graph, new lengths ---
def test_graph_replays_follow_new_lengths(gpu):
    """The lengths are read by the kernels at run time: a graph captured once
    is replayed after the length arrays change, and each replay matches the
    oracle for the lengths it saw."""
    wc = workloads.gen_prefill_chunked(2, 8, 2, 96, [1000, 1000], kv_cap=1000, seed=45)
    wd = workloads.gen_decode_gqa(3, 16, 4, D=128, kv_cap=2000, kv_lens=[2000] * 3, seed=46)
    wm = workloads.gen_decode_mla(2, 32, kv_cap=1500, kv_lens=[1500] * 2, seed=47)
    cq, ck, cv = dev_bf16(wc.q), dev_bf16(wc.k), dev_bf16(wc.v)
    dq, dk, dv = dev_bf16(wd.q), dev_bf16(wd.k), dev_bf16(wd.v)
    mq, mc = dev_bf16(wm.q), dev_bf16(wm.ckv)
    lc, ld, lm = _lens([1000, 1000]), _lens([2000] * 3), _lens([1500] * 2)
    oc, lsc = torch.empty_like(cq), torch.empty((2, 8, 96), device="cuda")
    od, lsd = torch.empty_like(dq), torch.empty((3, 16), device="cuda")
    om, lsm = torch.empty((2, 32, 512), dtype=torch.bfloat16, device="cuda"), torch.empty((2, 32), device="cuda")
    ws_d = torch.empty(gpu.attn_decode_gqa_workspace_bytes(3, 16, 4, 2000), dtype=torch.uint8, device="cuda")
    ws_m = torch.empty(gpu.attn_decode_mla_ragged_workspace_bytes(2, 32, 1500), dtype=torch.uint8,
                       device="cuda")

    def calls():
        gpu.attn_prefill_chunked(cq, ck, cv, lc, wc.scale, out=oc, lse=lsc)
        gpu.attn_decode_gqa_ragged(dq, dk, dv, ld, 2000, wd.scale, out=od, lse=lsd, ws=ws_d)
        gpu.attn_decode_mla_ragged(mq, mc, lm, 1500, wm.Dv, wm.scale, out=om, lse=lsm, ws=ws_m)

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for new_c, new_d, new_m in (([96, 1000], [2000, 1, 777], [1500, 9]),
                                ([500, 97], [0, 64, 1999], [600, 1200])):
        lc.copy_(_lens(new_c))
        ld.copy_(_lens(new_d))
        lm.copy_(_lens(new_m))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.prefill_chunked(wc.q, wc.k, wc.v, new_c, wc.scale)
        check_bf16(host(oc), o_ref, host(lsc), l_ref, "graph chunked %s" % (new_c,))
        o_ref, l_ref = oracle.decode_gqa_ragged(wd.q, wd.k, wd.v, new_d, wd.scale)
        _check_ragged(od, lsd, o_ref, l_ref, new_d, "graph gqa %s" % (new_d,))
        o_ref, l_ref = oracle.decode_mla_ragged(wm.q, wm.ckv, new_m, wm.Dv, wm.scale)
        _check_ragged(om, lsm, o_ref, l_ref, new_m, "graph mla %s" % (new_m,))
