"""GQA and absorbed-MLA decode on the GPU (through the C ABI) against the
fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_bf16, check_bf16_channels, dev_bf16, host

pytestmark = pytest.mark.gpu


def _gqa(gpu, w, ws=None):
    o, lse = gpu.attn_decode_gqa(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), w.kv_len, w.scale,
                                 ws=ws)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("B,Hq,Hkv,kv_len,kv_cap", [
    (1, 4, 1, 1, 8), (2, 8, 2, 5, 64), (2, 32, 8, 255, 300), (1, 8, 8, 256, 256),
    (3, 16, 4, 257, 512), (2, 32, 8, 1000, 1024), (1, 16, 1, 4095, 4100),
    (1, 32, 2, 3000, 3000), (4, 24, 8, 777, 800), (1, 2, 1, 70000, 70001), (8, 32, 8, 2, 8),
    (4, 32, 8, 3, 3)])
def test_decode_gqa_matches_oracle(gpu, B, Hq, Hkv, kv_len, kv_cap):
    """Ragged lengths, every group size 1..16 (3 is padded to 4), one and many
    splits; slots past kv_len hold NaN and must never be read."""
    w = workloads.gen_decode_gqa(B, Hq, Hkv, kv_len, D=128, kv_cap=kv_cap, seed=kv_len + Hq,
                                 poison_tail=True)
    o, lse = _gqa(gpu, w)
    o_ref, lse_ref = oracle.decode_gqa(w.q, w.k, w.v, w.kv_len, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "gqa %s" % ((B, Hq, Hkv, kv_len),))


def test_decode_gqa_llama3_workload_and_repeat(gpu):
    """The Llama-3-8B-shaped workload in full (B=8, 32/8 heads, 4096 keys);
    three calls reusing one workspace give bit-identical results (the split
    counters reset themselves)."""
    w = workloads.make("decode_gqa_llama3_8b_4k")
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    outs = [gpu.attn_decode_gqa(q, k, v, w.kv_len, w.scale) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])
    o_ref, lse_ref = oracle.decode_gqa(w.q, w.k, w.v, w.kv_len, w.scale)
    check_bf16(host(outs[0][0]), o_ref, host(outs[0][1]), lse_ref, "decode_gqa_llama3_8b_4k")


def test_decode_gqa_workspace_contents_do_not_matter(gpu):
    """Nothing in the workspace is read before the call writes it: a
    workspace holding random bytes, all ones, zeros, or what a call of
    another shape left in it gives the same bits as a fresh one, call after
    call."""
    w = workloads.gen_decode_gqa(2, 32, 8, 3000, D=128, kv_cap=3072, seed=5)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    o_ref, l_ref = gpu.attn_decode_gqa(q, k, v, w.kv_len, w.scale)
    need = gpu.attn_decode_gqa_workspace_bytes(2, 32, 8, 3000)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    w2 = workloads.gen_decode_gqa(1, 8, 2, 2000, D=128, seed=6)
    gen = torch.Generator().manual_seed(7)
    for fill in ("random", "ones", "zeros", "other call"):
        if fill == "random":
            ws.copy_(torch.randint(0, 256, (need,), generator=gen, dtype=torch.uint8))
        elif fill == "ones":
            ws.fill_(255)
        elif fill == "zeros":
            ws.zero_()
        else:
            gpu.attn_decode_gqa(dev_bf16(w2.q), dev_bf16(w2.k), dev_bf16(w2.v), w2.kv_len, w2.scale,
                                ws=ws)
        for rep in range(2):
            o, l = gpu.attn_decode_gqa(q, k, v, w.kv_len, w.scale, ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), (fill, rep)
            assert torch.equal(l, l_ref), (fill, rep)
    o_or, l_or = oracle.decode_gqa(w.q, w.k, w.v, w.kv_len, w.scale)
    check_bf16(host(o_ref), o_or, host(l_ref), l_or, "gqa workspace")


def test_decode_matches_prefill_rows(gpu):
    """A cached decode step for token t equals row t of a causal prefill over
    the same tokens (earlier rows never see later tokens)."""
    w = workloads.gen_prefill(1, 8, 2, 300, 128, dtype="bf16", seed=12)
    o_p, l_p = gpu.attn_prefill_causal(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), w.scale)
    for t in (0, 1, 63, 64, 299):
        o_d, l_d = gpu.attn_decode_gqa(dev_bf16(w.q[:, :, t]), dev_bf16(w.k), dev_bf16(w.v), t + 1,
                                       w.scale)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.prefill_causal(w.q, w.k, w.v, w.scale, rows=[t])
        check_bf16(host(o_d), o_ref[:, :, 0], host(l_d), l_ref[:, :, 0], "decode t=%d" % t)
        check_bf16(host(o_d), host(o_p[:, :, t]), host(l_d), host(l_p[:, :, t]), "vs prefill t=%d" % t)


def _mla(gpu, w):
    o, lse = gpu.attn_decode_mla_absorbed(dev_bf16(w.q), dev_bf16(w.ckv), w.kv_len, w.Dv, w.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("B,Hq,kv_len,kv_cap", [
    (1, 16, 1, 32), (4, 128, 2, 8), (2, 64, 3, 3), (2, 16, 31, 64), (1, 128, 33, 40),
    (2, 32, 1000, 1024), (1, 128, 5000, 5000), (1, 144, 70, 100),
    (260, 16, 545, 560),   # one split per sequence (no merge), pipelined loop, partial tile
    (2, 256, 600, 608)])   # two head groups, one tile per split
def test_decode_mla_matches_oracle(gpu, B, Hq, kv_len, kv_cap):
    w = workloads.gen_decode_mla(B, Hq, kv_len, kv_cap=kv_cap, seed=kv_len + Hq)
    o, lse = _mla(gpu, w)
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q, w.ckv, w.kv_len, w.Dv, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "mla %s" % ((B, Hq, kv_len),))


def test_decode_mla_32k_workload_sampled_batches(gpu):
    """The full MLA workload (B=16, 128 heads, 32768 latent rows of 576,
    balanced channels); every output finite; the oracle checks two batches."""
    w = workloads.make("decode_mla_absorbed_32k")
    o, lse = _mla(gpu, w)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    bs = [0, w.B - 1]
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q[bs], w.ckv[bs], w.kv_len, w.Dv, w.scale)
    check_bf16(host(o[bs]), o_ref, host(lse[bs]), lse_ref, "decode_mla_absorbed_32k")


def test_decode_mla_raw_latent_32k_sampled_batches(gpu):
    """The MLA workload's shape (B=16, 128 heads, 32768 latent rows of 576)
    with the absorbed query and latent stored raw, without the channel scale:
    query channels of magnitude 1e-4..1e2, latent channels the reciprocals
    (up to ~4e4). fp32 accumulation is what keeps the scores right here
    ("MLA 矩阵乘法吸收的数值稳定性治理", §二.2, §五). Two batches against the
    oracle, channel by channel in units of each channel's values."""
    w = workloads.make("decode_mla_absorbed_32k", balance=False)
    o, lse = _mla(gpu, w)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    bs = [0, w.B - 1]
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q[bs], w.ckv[bs], w.kv_len, w.Dv, w.scale)
    vals = oracle.widen(w.ckv[bs][:, :w.kv_len, :w.Dv])
    check_bf16_channels(host(o[bs]), o_ref, host(lse[bs]), lse_ref, vals, "mla raw latent 32k")


@pytest.mark.parametrize("B,Hq,kv_len", [(1, 128, 4096), (2, 64, 700), (3, 32, 1)])
def test_decode_mla_values_beyond_fp16_range(gpu, B, Hq, kv_len):
    """Latent channels of magnitude 1e5..1e6 (raw storage, query channels
    1e-6..1e-5): the values exceed fp16's largest finite 65504, which bf16
    holds. Split partials, the merge and the single-split path all keep
    them (a 16-bit float partial would give Inf), and the output is rounded
    once. Uniform and ragged calls."""
    w = workloads.gen_decode_mla(B, Hq, kv_len, kv_cap=kv_len + 3, seed=kv_len + Hq,
                                 balance=False, mag_lo=1e-6, mag_hi=1e-5)
    vals = oracle.widen(w.ckv[:, :kv_len, :w.Dv])
    assert np.abs(vals).max() > 65504
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q, w.ckv, kv_len, w.Dv, w.scale)
    q, c = dev_bf16(w.q), dev_bf16(w.ckv)
    o, lse = gpu.attn_decode_mla_absorbed(q, c, kv_len, w.Dv, w.scale)
    lens = torch.full((B,), kv_len, dtype=torch.int32, device="cuda")
    o2, lse2 = gpu.attn_decode_mla_ragged(q, c, lens, kv_len, w.Dv, w.scale)
    torch.cuda.synchronize()
    assert np.abs(host(o)).max() > 65504
    check_bf16_channels(host(o), o_ref, host(lse), lse_ref, vals, "mla |v| > 65504 %s" % ((B, Hq, kv_len),))
    check_bf16_channels(host(o2), o_ref, host(lse2), lse_ref, vals, "ragged mla |v| > 65504")


@pytest.mark.parametrize("kv_len", [512, 513])
def test_decode_mla_weight_residual_cutoff(gpu, kv_len):
    """Caches of up to 512 keys add the product with the bf16 residual of the
    weights; longer caches use bf16 weights alone. Both sides of the cut meet
    the bar."""
    w = workloads.gen_decode_mla(2, 64, kv_len, kv_cap=kv_len + 7, seed=kv_len)
    o, lse = _mla(gpu, w)
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q, w.ckv, w.kv_len, w.Dv, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "mla cutoff kv_len=%d" % kv_len)


@pytest.mark.parametrize("B,kv_len,ramp,climb", [(1, 300, 48.0, 24), (1, 1500, 48.0, 24),
                                                 (16, 2048, 2000.0, 40)])
def test_decode_mla_rising_scores(gpu, B, kv_len, ramp, climb):
    """The rope channels of the latent rows (part of each key, not of its
    value) are scaled up with the row's position, ×1 → ×ramp: the scores of
    later tiles exceed the running maximum again and again, and the softmax
    ends up dominated by a few late keys while the values stay O(1). With the
    steep ramp the scores climb by more than `climb` log2 units within a
    single split of the cache (16 sequences: 16 splits of 128 keys), many
    times the 8 log2 units the kernel's reference may lag the running maximum
    before the output is rescaled, so the rescale runs again and again inside
    one split. Slots past kv_len stay NaN."""
    w = workloads.gen_decode_mla(B, 32, kv_len, kv_cap=kv_len + 5, seed=9)
    x = oracle.widen(w.ckv[:, :kv_len])
    x[..., w.Dv:] *= np.linspace(1.0, ramp, kv_len)[None, :, None]
    w.ckv[:, :kv_len] = workloads.round_to_bf16_bits(x)
    o, lse = _mla(gpu, w)
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q, w.ckv, w.kv_len, w.Dv, w.scale)
    s = oracle.widen(w.q[0]) @ oracle.widen(w.ckv[0, :kv_len]).T * w.scale / np.log(2.0)
    per = kv_len if B == 1 else kv_len // (256 // B)   # keys of one split of sequence 0
    assert (s[:, per - 32:per].max(axis=1) - s[:, :32].max(axis=1)).min() > climb
    check_bf16(host(o), o_ref, host(lse), lse_ref, "mla rising scores kv_len=%d ramp=%g" % (kv_len, ramp))


# ------------------------------------------------------------ FP8 E4M3 cache ---
def _dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


@pytest.mark.parametrize("B,Hq,Hkv,kv_len,kv_cap", [
    (1, 4, 1, 1, 8), (2, 8, 2, 5, 64), (2, 32, 8, 255, 300), (3, 16, 4, 257, 512),
    (1, 16, 1, 4095, 4100), (4, 24, 8, 777, 800), (1, 2, 1, 70000, 70001), (8, 32, 8, 2, 8)])
def test_decode_gqa_fp8_matches_oracle(gpu, B, Hq, Hkv, kv_len, kv_cap):
    """E4M3 caches (the NaN code fills the slots past kv_len): the kernel
    converts the stored codes exactly, so the oracle over the same codes is
    the reference."""
    w = workloads.gen_decode_gqa(B, Hq, Hkv, kv_len, D=128, kv_cap=kv_cap, seed=kv_len + 3 * Hq,
                                 cache_dtype="fp8")
    o, lse = gpu.attn_decode_gqa_fp8(dev_bf16(w.q), _dev_u8(w.k), _dev_u8(w.v), kv_len, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_gqa(w.q, w.k, w.v, kv_len, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "gqa fp8 %s" % ((B, Hq, Hkv, kv_len),))


def test_decode_gqa_fp8_workload_equals_bf16_copy_of_its_values(gpu):
    """The Llama-3-8B decode over an E4M3 cache meets the bar, and so does
    the bf16 kernel run on the same values stored as bf16 (exact widening);
    the two differ only in the order the products are summed (the E4M3 path
    takes the head dimension in another order across the MFMA steps)."""
    w = workloads.make("decode_gqa_fp8_llama3_8b_4k")
    q = dev_bf16(w.q)
    o8, l8 = gpu.attn_decode_gqa_fp8(q, _dev_u8(w.k), _dev_u8(w.v), w.kv_len, w.scale)
    kb = workloads.round_to_bf16_bits(oracle.widen(w.k))
    vb = workloads.round_to_bf16_bits(oracle.widen(w.v))
    ob, lb = gpu.attn_decode_gqa(q, dev_bf16(kb), dev_bf16(vb), w.kv_len, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_gqa(w.q, w.k, w.v, w.kv_len, w.scale)
    check_bf16(host(o8), o_ref, host(l8), lse_ref, "decode_gqa_fp8_llama3_8b_4k")
    check_bf16(host(ob), o_ref, host(lb), lse_ref, "bf16 copy of the E4M3 values")


@pytest.mark.parametrize("B,Hq,kv_len,kv_cap", [
    (1, 16, 1, 32), (4, 128, 2, 8), (2, 64, 3, 3), (2, 16, 31, 64), (1, 128, 33, 40),
    (2, 64, 512, 520), (2, 64, 513, 520), (2, 32, 1000, 1024), (1, 128, 5000, 5000),
    (1, 144, 70, 100), (260, 16, 545, 560)])
def test_decode_mla_fp8_matches_oracle(gpu, B, Hq, kv_len, kv_cap):
    """E4M3 latent cache (balanced rows S·c, the NaN code past kv_len):
    partial tiles, 16..144 heads (partial head groups), one and many splits,
    both sides of the 512-key weight-residual cut. The oracle reads the same
    codes."""
    w = workloads.gen_decode_mla(B, Hq, kv_len, kv_cap=kv_cap, seed=kv_len + 5 * Hq,
                                 cache_dtype="fp8")
    o, lse = gpu.attn_decode_mla_fp8(dev_bf16(w.q), _dev_u8(w.ckv), kv_len, w.Dv, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q, w.ckv, kv_len, w.Dv, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "mla fp8 %s" % ((B, Hq, kv_len),))


def test_decode_mla_fp8_32k_workload(gpu):
    """The 32K MLA workload over an E4M3 cache: every output finite, two
    batches against the oracle, and the same bits as the bf16 kernel given a
    bf16 copy of the cached values (every E4M3 value is a bf16 value; the
    two paths feed the same operands to the same products in the same
    order, so this checks the E4M3 tile layout and its transposed reads
    element for element)."""
    w = workloads.make("decode_mla_fp8_32k")
    q = dev_bf16(w.q)
    o8, l8 = gpu.attn_decode_mla_fp8(q, _dev_u8(w.ckv), w.kv_len, w.Dv, w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o8.float()).all()) and bool(torch.isfinite(l8).all())
    c16 = torch.from_numpy(w.ckv).to("cuda").view(torch.float8_e4m3fn).to(torch.bfloat16)
    o16, l16 = gpu.attn_decode_mla_absorbed(q, c16, w.kv_len, w.Dv, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o8.view(torch.int16), o16.view(torch.int16))
    assert torch.equal(l8, l16)
    bs = [0, w.B - 1]
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q[bs], w.ckv[bs], w.kv_len, w.Dv, w.scale)
    check_bf16(host(o8[bs]), o_ref, host(l8[bs]), lse_ref, "decode_mla_fp8_32k")
