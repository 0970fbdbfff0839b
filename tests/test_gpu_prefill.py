"""Causal prefill on the GPU (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_bf16, check_f32, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu


def _run_bf16(gpu, w):
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    o, lse = gpu.attn_prefill_causal(q, k, v, w.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("B,Hq,Hkv,N,D", [
    (1, 2, 2, 64, 64), (1, 4, 2, 1, 64), (1, 4, 2, 17, 128), (2, 4, 1, 100, 64),
    (1, 2, 2, 129, 128), (1, 3, 1, 40, 128)])
def test_prefill_f32_matches_oracle(gpu, B, Hq, Hkv, N, D):
    w = workloads.gen_prefill(B, Hq, Hkv, N, D, dtype="f32", seed=100 + N)
    o, lse = gpu.attn_prefill_causal(dev_f32(w.q), dev_f32(w.k), dev_f32(w.v), w.scale)
    o_ref, lse_ref = oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    check_f32(host(o), o_ref, host(lse), lse_ref, "f32 %s" % ((B, Hq, Hkv, N, D),))


def test_prefill_f32_tiny_workload(gpu):
    """The named tiny workload: B=1, 2 heads, N=64, d=64, fp32, scale 1/8."""
    w = workloads.make("prefill_f32_tiny")
    o, lse = gpu.attn_prefill_causal(dev_f32(w.q), dev_f32(w.k), dev_f32(w.v), w.scale)
    assert o.shape == (1, 2, 64, 64) and lse.shape == (1, 2, 64) and o.dtype == torch.float32
    o_ref, lse_ref = oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    check_f32(host(o), o_ref, host(lse), lse_ref, "prefill_f32_tiny")


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 300])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_bf16_ragged_lengths(gpu, N, D):
    w = workloads.gen_prefill(1, 8, 2, N, D, dtype="bf16", seed=7 * N + D)
    o, lse = _run_bf16(gpu, w)
    o_ref, lse_ref = oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "bf16 N=%d D=%d" % (N, D))


@pytest.mark.parametrize("B,Hq,Hkv,N", [(2, 4, 4, 257), (1, 16, 2, 1000), (3, 6, 3, 130)])
def test_prefill_bf16_gqa_groups(gpu, B, Hq, Hkv, N):
    w = workloads.gen_prefill(B, Hq, Hkv, N, 128, dtype="bf16", seed=B * 1000 + N)
    o, lse = _run_bf16(gpu, w)
    o_ref, lse_ref = oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "bf16 %s" % ((B, Hq, Hkv, N),))


def test_prefill_bf16_row0_is_v0_and_deterministic(gpu):
    """Query 0 sees only key 0: O[0] = V[0] exactly (one weight of 1, one
    rounding of an already-bf16 value). Two runs agree bit for bit."""
    w = workloads.gen_prefill(2, 8, 2, 700, 128, dtype="bf16", seed=3)
    o1, l1 = _run_bf16(gpu, w)
    o2, l2 = _run_bf16(gpu, w)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    v = dev_bf16(w.v)
    for hq in range(8):
        assert torch.equal(o1[:, hq, 0].view(torch.int16), v[:, hq // 4, 0].view(torch.int16))


def _sample_rows(N, rng, extra=()):
    rows = {0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 256, N // 2, N - 2, N - 1}
    rows |= set(int(r) for r in rng.choice(N, 10, replace=False))
    rows |= {int(r) for r in extra if 0 <= r < N}
    return np.array(sorted(rows), dtype=np.int32)


def test_prefill_bf16_4k_workload_sampled_rows(gpu):
    """The B=4, 32/8 heads, N=4096, d=128 workload at full size; the oracle
    checks a sample of rows of every (b, head); every output is finite."""
    w = workloads.make("prefill_bf16_4k")
    o, lse = _run_bf16(gpu, w)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    rows = _sample_rows(w.N, np.random.default_rng(0))
    o_ref, lse_ref = oracle.prefill_causal(w.q, w.k, w.v, w.scale, rows=rows)
    check_bf16(host(o[:, :, rows]), o_ref, host(lse[:, :, rows]), lse_ref, "prefill_bf16_4k")


def test_prefill_bf16_32k_outliers_sampled_rows(gpu):
    """N=32768 with 1 % of K rows scaled ×8 (outlier logits force running-max
    jumps); rows include those sitting on outlier keys and just after."""
    w = workloads.make("prefill_bf16_32k_outliers")
    o, lse = _run_bf16(gpu, w)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    outl = w.outlier_rows[0, 0]
    rows = _sample_rows(w.N, np.random.default_rng(1), extra=list(outl[:6]) + list(outl[:6] + 1))
    o_ref, lse_ref = oracle.prefill_causal(w.q, w.k, w.v, w.scale, rows=rows)
    check_bf16(host(o[:, :, rows]), o_ref, host(lse[:, :, rows]), lse_ref, "prefill_bf16_32k")
