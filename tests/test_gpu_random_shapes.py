"""Seeded random shapes through every decode and prefill entry point, against
the fp64 oracle: a sweep beside the hand-picked cases, drawn once from a
fixed generator so every run sees the same shapes. Sizes stay small enough
for the oracle (each case well under a second on the host)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_bf16, check_f32, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu

_R = np.random.default_rng(20261203)


def _lens(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device="cuda")


def _u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _gqa_cases(n):
    out = []
    for _ in range(n):
        Hkv = int(_R.choice([1, 2, 4, 8]))
        G = int(_R.choice([1, 2, 4, 8]))
        B = int(_R.integers(1, 5))
        kv_len = int(_R.integers(1, 3000))
        kv_cap = kv_len + int(_R.integers(0, 64))
        out.append((B, G * Hkv, Hkv, kv_len, kv_cap))
    return out


def _mla_cases(n):
    out = []
    for _ in range(n):
        B = int(_R.integers(1, 4))
        Hq = 16 * int(_R.integers(1, 11))          # 16 .. 160 heads, partial head groups
        kv_len = int(_R.integers(1, 2500))
        kv_cap = kv_len + int(_R.integers(0, 40))
        out.append((B, Hq, kv_len, kv_cap))
    return out


def _prefill_cases(n):
    out = []
    for _ in range(n):
        D = int(_R.choice([64, 128]))
        Hkv = int(_R.choice([1, 2, 4]))
        G = int(_R.choice([1, 2, 4]))
        B = int(_R.integers(1, 3))
        N = int(_R.integers(1, 700))
        out.append((B, G * Hkv, Hkv, N, D))
    return out


@pytest.mark.parametrize("B,Hq,Hkv,kv_len,kv_cap", _gqa_cases(8))
def test_random_decode_gqa(gpu, B, Hq, Hkv, kv_len, kv_cap):
    w = workloads.gen_decode_gqa(B, Hq, Hkv, kv_len, kv_cap=kv_cap, seed=kv_len + Hq)
    o, lse = gpu.attn_decode_gqa(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), kv_len, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_gqa(w.q, w.k, w.v, kv_len, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "gqa %s" % ((B, Hq, Hkv, kv_len),))


@pytest.mark.parametrize("B,Hq,Hkv,kv_len,kv_cap,lens", [
    c + ([int(x) for x in _R.integers(1, c[3] + 1, size=c[0])],) for c in _gqa_cases(6)])
def test_random_decode_gqa_fp8_ragged(gpu, B, Hq, Hkv, kv_len, kv_cap, lens):
    """An E4M3 uniform call, then the ragged bf16 entry point on seeded lengths."""
    w = workloads.gen_decode_gqa(B, Hq, Hkv, kv_len, kv_cap=kv_cap, seed=kv_len + 3, cache_dtype="fp8")
    o, lse = gpu.attn_decode_gqa_fp8(dev_bf16(w.q), _u8(w.k), _u8(w.v), kv_len, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_gqa(w.q, w.k, w.v, kv_len, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "gqa fp8 %s" % ((B, Hq, Hkv, kv_len),))
    wr = workloads.gen_decode_gqa(B, Hq, Hkv, D=128, kv_cap=kv_cap, kv_lens=lens, seed=kv_len + 4)
    o, lse = gpu.attn_decode_gqa_ragged(dev_bf16(wr.q), dev_bf16(wr.k), dev_bf16(wr.v), _lens(lens),
                                        max(lens), wr.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_gqa_ragged(wr.q, wr.k, wr.v, wr.kv_lens, wr.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "gqa ragged %s" % (lens,))


@pytest.mark.parametrize("B,Hq,kv_len,kv_cap,lens", [
    c + ([int(x) for x in _R.integers(0, c[2] + 1, size=c[0])],) for c in _mla_cases(8)])
def test_random_decode_mla(gpu, B, Hq, kv_len, kv_cap, lens):
    """bf16 and E4M3 latent caches, uniform and ragged, on the same shape."""
    w = workloads.gen_decode_mla(B, Hq, kv_len, kv_cap=kv_cap, seed=kv_len + Hq)
    o, lse = gpu.attn_decode_mla_absorbed(dev_bf16(w.q), dev_bf16(w.ckv), kv_len, w.Dv, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_mla_absorbed(w.q, w.ckv, kv_len, w.Dv, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "mla %s" % ((B, Hq, kv_len),))
    w8 = workloads.gen_decode_mla(B, Hq, kv_len, kv_cap=kv_cap, seed=kv_len + 1, cache_dtype="fp8")
    o, lse = gpu.attn_decode_mla_fp8(dev_bf16(w8.q), _u8(w8.ckv), kv_len, w8.Dv, w8.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_mla_absorbed(w8.q, w8.ckv, kv_len, w8.Dv, w8.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "mla fp8 %s" % ((B, Hq, kv_len),))
    if max(lens) > 0:
        wr = workloads.gen_decode_mla(B, Hq, kv_cap=kv_cap, kv_lens=lens, seed=kv_len + 2,
                                      cache_dtype="fp8")
        o, lse = gpu.attn_decode_mla_ragged_fp8(dev_bf16(wr.q), _u8(wr.ckv), _lens(lens), max(lens),
                                                wr.Dv, wr.scale)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.decode_mla_ragged(wr.q, wr.ckv, wr.kv_lens, wr.Dv, wr.scale)
        full = np.flatnonzero(np.asarray(lens) > 0)
        check_bf16(host(o)[full], o_ref[full], host(lse)[full], lse_ref[full],
                   "mla ragged fp8 %s" % (lens,))


@pytest.mark.parametrize("B,Hq,Hkv,N,D", _prefill_cases(8))
def test_random_prefill(gpu, B, Hq, Hkv, N, D):
    """bf16 and fp32 causal prefill on the same shape."""
    w = workloads.gen_prefill(B, Hq, Hkv, N, D, dtype="bf16", seed=N + D)
    o, lse = gpu.attn_prefill_causal(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "prefill bf16 %s" % ((B, Hq, Hkv, N, D),))
    w = workloads.gen_prefill(B, Hq, Hkv, N, D, dtype="f32", seed=N + D + 1)
    o, lse = gpu.attn_prefill_causal(dev_f32(w.q), dev_f32(w.k), dev_f32(w.v), w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    check_f32(host(o), o_ref, host(lse), lse_ref, "prefill f32 %s" % ((B, Hq, Hkv, N, D),))


def _chunked_cases(n):
    out = []
    for _ in range(n):
        Hkv = int(_R.choice([1, 2, 4]))
        G = int(_R.choice([1, 2, 4]))
        B = int(_R.integers(1, 3))
        N = int(_R.integers(1, 260))
        hist = [int(x) for x in _R.integers(0, 900, size=B)]
        out.append((B, G * Hkv, Hkv, N, hist))
    return out


@pytest.mark.parametrize("B,Hq,Hkv,N,hist", _chunked_cases(6))
def test_random_prefill_chunked(gpu, B, Hq, Hkv, N, hist):
    """A chunk of N queries against a cache with a seeded history per sequence (d = 128)."""
    lens = [N + h for h in hist]
    w = workloads.gen_prefill_chunked(B, Hq, Hkv, N, lens, kv_cap=max(lens) + 8, seed=N + 9)
    o, lse = gpu.attn_prefill_chunked(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), _lens(lens),
                                      w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.prefill_chunked(w.q, w.k, w.v, w.kv_lens, w.scale)
    check_bf16(host(o), o_ref, host(lse), lse_ref, "chunked %s" % ((B, Hq, Hkv, N, lens),))
