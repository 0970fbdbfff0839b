"""Seeded generators: storage rounding, determinism, workload structure."""
import numpy as np
import torch

import oracle
import workloads


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e-39, 65504.0])])
    ours = workloads.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = workloads.bf16_bits_as_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic():
    a = workloads.gen_prefill(1, 4, 2, 33, 16, seed=5)
    b = workloads.gen_prefill(1, 4, 2, 33, 16, seed=5)
    c = workloads.gen_prefill(1, 4, 2, 33, 16, seed=6)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a.q, c.q)


def test_outlier_rows_are_exactly_scaled():
    base = workloads.gen_prefill(1, 4, 2, 1000, 32, seed=9)
    out = workloads.gen_prefill(1, 4, 2, 1000, 32, seed=9, outlier_frac=0.01, outlier_mult=8.0)
    assert out.outlier_rows.shape == (1, 2, 10)
    for h in range(2):
        sel = out.outlier_rows[0, h]
        assert len(set(sel.tolist())) == 10
        kb = workloads.bf16_bits_as_f32(base.k[0, h])
        ko = workloads.bf16_bits_as_f32(out.k[0, h])
        np.testing.assert_array_equal(ko[sel], kb[sel] * 8)
        rest = np.setdiff1d(np.arange(1000), sel)
        np.testing.assert_array_equal(ko[rest], kb[rest])
    np.testing.assert_array_equal(out.q, base.q)


def test_decode_poison_tail():
    w = workloads.gen_decode_gqa(2, 8, 2, 100, D=64, kv_cap=128, seed=1)
    assert np.all(w.k[:, :, 100:] == workloads.BF16_NAN_BITS)
    assert np.all(np.isfinite(workloads.bf16_bits_as_f32(w.k[:, :, :100])))


def test_mla_balanced_storage_is_unit_range():
    """Channel balancing leaves the stored latent channels near unit scale
    even though the model-side magnitudes span 1e-4..1e2. S is estimated from
    calibration draws, not copied from the true magnitudes, so the stored
    channels keep some imbalance (a few per cent to a few tens of per cent)."""
    w = workloads.gen_decode_mla(1, 8, 256, seed=3)
    assert w.mags.min() >= 1e-4 and w.mags.max() <= 1e2
    assert np.log10(w.mags.max() / w.mags.min()) > 4
    ratio = w.s / w.mags
    assert 0.6 < ratio.min() and ratio.max() < 1.6 and np.abs(ratio - 1).max() > 0.05
    c = workloads.bf16_bits_as_f32(w.ckv[0, :256, :512])
    rms = np.sqrt((c.astype(np.float64) ** 2).mean(0))
    assert 0.5 < rms.min() and rms.max() < 2.0


def test_mla_raw_storage_keeps_channel_magnitudes():
    """balance=False stores the model-side q̃ and c themselves: query channel
    magnitudes span 1e-4..1e2 and the latent's their reciprocals (a channel
    of magnitude 1e-6 puts latent values far beyond fp16's 65504, which
    bf16 holds)."""
    w = workloads.gen_decode_mla(1, 64, 512, seed=3, balance=False)
    assert np.all(w.s == 1.0)
    q = workloads.bf16_bits_as_f32(w.q[0, :, :512]).astype(np.float64)
    c = workloads.bf16_bits_as_f32(w.ckv[0, :, :512]).astype(np.float64)
    rq = np.sqrt((q ** 2).mean(0)) / w.mags
    rc = np.sqrt((c ** 2).mean(0)) * w.mags
    assert 0.6 < rq.min() and rq.max() < 1.6 and 0.8 < rc.min() and rc.max() < 1.25
    big = workloads.gen_decode_mla(1, 16, 64, seed=5, balance=False, mag_lo=1e-6, mag_hi=1e-5)
    assert np.abs(workloads.bf16_bits_as_f32(big.ckv[0, :, :512])).max() > 65504


def test_named_workload_shapes():
    assert workloads.WORKLOADS["decode_gqa_llama3_8b_4k"]["Hq"] == 32
    w = workloads.make("decode_gqa_llama3_8b_4k", B=1, kv_len=64)
    assert w.q.shape == (1, 32, 128) and w.k.shape == (1, 8, 64, 128)
    # algorithmic bytes of the full GQA decode workload
    assert workloads.decode_gqa_bytes(8, 32, 8, 4096, 128) == 134_349_824
    assert workloads.prefill_causal_flops(4, 32, 4096, 128) == 549_890_031_616
    assert workloads.decode_mla_bytes(16, 128, 32768, 576, 512) == 608_444_416


def test_e4m3_rounding_matches_torch_in_range():
    """FP8 E4M3 storage rounding (nearest, ties to even) agrees with torch's
    float8_e4m3fn conversion for every magnitude up to 448, including the
    exact midpoints between codes; larger magnitudes saturate to ±448."""
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000) * 4, rng.uniform(-448, 448, 20000),
                        [0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11, 1.0625, 1.1875, 448.0, -448.0]])
    x = x.astype(np.float32)
    ours = workloads.round_to_e4m3_bits(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)
    # midpoints between neighbouring codes go to the even code
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    codes = workloads.round_to_e4m3_bits(mids)
    assert np.all(codes % 2 == 0)
    np.testing.assert_array_equal(workloads.round_to_e4m3_bits(np.array([500.0, -1e9, 464.0])),
                                  np.array([0x7E, 0xFE, 0x7E], np.uint8))


def test_fp8_decode_cache_poison_and_dtype():
    w = workloads.gen_decode_gqa(2, 4, 2, 10, D=16, kv_cap=12, seed=3, cache_dtype="fp8")
    assert w.k.dtype == np.uint8 and w.v.dtype == np.uint8 and w.q.dtype == np.uint16
    assert np.all(w.k[:, :, 10:] == workloads.E4M3_NAN_BITS)
    assert np.all(w.k[:, :, :10] != workloads.E4M3_NAN_BITS)


def test_channel_scale_makes_latent_fit_e4m3():
    """The static channel scale S is what lets the MLA latent live in E4M3
    ("MLA 矩阵乘法吸收的数值稳定性治理", §二.1). The raw latent c (channel
    magnitudes over six decades) overflows E4M3's largest finite value, 448,
    in a large share of its entries; the balanced S·c that is stored never
    does, and every balanced entry in E4M3's normal range (≥ 2^-6) keeps a
    relative error of at most 2^-4 (3 mantissa bits, round to nearest)."""
    w = workloads.gen_decode_mla(1, 16, 2000, seed=4)
    bal = oracle.widen(w.ckv[0, :, :w.Dv])      # stored S·c (bf16)
    raw = bal / w.s                              # the model's latent c
    assert np.mean(np.abs(raw) > 448.0) > 0.1
    assert np.abs(bal).max() < 448.0
    q = oracle.widen(workloads.round_to_e4m3_bits(bal))
    normal = np.abs(bal) >= 2.0 ** -6
    assert normal.mean() > 0.98          # N(0,1): about 1.2 % lie below 2^-6
    assert np.all(np.abs(q - bal)[normal] <= 2.0 ** -4 * np.abs(bal)[normal])
    # the E4M3 generator rounds the same balanced draws (from fp64, so within
    # half an E4M3 step of them, plus the bf16 copy's own rounding)
    w8 = workloads.gen_decode_mla(1, 16, 2000, seed=4, cache_dtype="fp8")
    q8 = oracle.widen(w8.ckv[0, :, :w.Dv])
    assert np.all(np.abs(q8 - bal) <= 2.0 ** -4 * np.abs(bal) + 2.0 ** -10)
