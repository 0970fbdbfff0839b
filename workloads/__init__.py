"""Seeded synthetic inputs for the attention hot path.

This module is shared by the CPU oracle (tests, bench baseline) and the GPU
path. It holds no attention arithmetic: only random draws, storage rounding
to bfloat16, the fixed shapes of the five workloads, and the algorithmic
flop / byte counts used to price a launch against a roofline.

Every array is drawn with numpy's PCG64 from a fixed seed. Inputs are N(0,1)
draws in float32, rounded once to bfloat16 with round-to-nearest-even when
the workload stores bf16. bf16 arrays are returned as their raw uint16 bit
patterns, so both sides start from exactly the same stored values.

Workload shapes follow the pages:
  * 05 · Tích vô hướng, Softmax và toán của Attention (inference-notes), §4:
    Llama-3-8B decode, 32 query heads sharing 8 K/V heads, d=128, 4096-token
    context, 128 KiB of K/V per token.
  * MLA 矩阵乘法吸收的数值稳定性治理 (gsyq.cn), §一 and §二.1: 512-dim latent
    cache, per-channel magnitudes spanning 1e-4..1e2, a static diagonal
    channel scale S applied as q·S⁻¹ and S·c.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)


# ---------------------------------------------------------------- storage ---
def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 (or float64) values to bfloat16, nearest-even; return bits.

    Inputs must be finite. float64 is first rounded to float32; the draws
    here are float32 already, so that step is exact for them.
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


# OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
# infinity; S.1111.111 is NaN; largest finite 448, smallest subnormal 2^-9).
E4M3_NAN_BITS = np.uint8(0x7F)


def _e4m3_magnitudes() -> np.ndarray:
    """Values of the finite non-negative codes 0x00..0x7E, increasing."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))


def round_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round finite values to FP8 E4M3 codes: nearest, ties to the even code,
    magnitudes above 448 saturate to 448."""
    x = np.asarray(x, dtype=np.float64)
    vals = _e4m3_magnitudes()
    a = np.minimum(np.abs(x), 448.0)
    i = np.clip(np.searchsorted(vals, a), 1, 126)
    lo, hi = vals[i - 1], vals[i]
    up = (a - lo > hi - a) | ((a - lo == hi - a) & (i % 2 == 0))
    code = np.where(up, i, i - 1).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << np.uint8(7))


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _rng(seed: int, n_children: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n_children)]


def _normal(rng, shape, chunk=1 << 24) -> np.ndarray:
    """N(0,1) float32 draws, generated in chunks to bound peak memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def _normal_e4m3(rng, shape, chunk=1 << 22) -> np.ndarray:
    """N(0,1) float32 draws stored as FP8 E4M3 codes."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = round_to_e4m3_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def _normal_bf16(rng, shape, chunk=1 << 24) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = round_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


# -------------------------------------------------------------- workloads ---
@dataclass
class Prefill:
    """Causal prefill inputs. q [B,Hq,N,D]; k, v [B,Hkv,N,D]; D innermost."""
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    dtype: str            # "bf16" (uint16 bits) or "f32"
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    outlier_rows: np.ndarray | None = None   # [B,Hkv,n_out] key rows scaled ×8


@dataclass
class DecodeGQA:
    """Single-query GQA decode. q [B,Hq,D]; k_cache, v_cache [B,Hkv,kv_cap,D] bf16."""
    B: int
    Hq: int
    Hkv: int
    kv_len: int
    kv_cap: int
    D: int
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    kv_lens: np.ndarray | None = None   # [B] int32 per-sequence lengths (ragged batch)
    cache_dtype: str = "bf16"           # "bf16" (uint16 bits) or "fp8" (E4M3 uint8 codes)


@dataclass
class PrefillChunked:
    """A chunk of Nq new tokens per sequence attending to a K/V cache.

    q [B,Hq,Nq,D]; k, v [B,Hkv,kv_cap,D] bf16. Sequence b has kv_lens[b]
    filled slots; the last Nq of them are the chunk's own K/V (already
    appended), the ones before are its history.
    """
    B: int
    Hq: int
    Hkv: int
    Nq: int
    kv_cap: int
    D: int
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    kv_lens: np.ndarray                 # [B] int32, each in [Nq, kv_cap]


@dataclass
class DecodeMLA:
    """Absorbed MLA decode. q [B,Hq,Dqk] bf16; ckv [B,kv_cap,Dqk] bf16 or
    FP8 E4M3 codes.

    Each row is [latent (Dv) | rope (Dqk-Dv)]. The latent part is stored
    channel-balanced (q holds q̃·S⁻¹ and ckv holds S·c, S = diag(s)) or raw
    (s = 1). V is the latent part of ckv (its first Dv channels).
    """
    B: int
    Hq: int
    kv_len: int
    kv_cap: int
    Dqk: int
    Dv: int
    scale: float
    q: np.ndarray
    ckv: np.ndarray
    s: np.ndarray = field(default=None)   # channel scale S applied before storage, [Dv] float64
    kv_lens: np.ndarray | None = None     # [B] int32 per-sequence lengths (ragged batch)
    cache_dtype: str = "bf16"             # "bf16" (uint16 bits) or "fp8" (E4M3 uint8 codes)
    mags: np.ndarray = field(default=None)  # true channel magnitudes of the raw q̃, [Dv]


def ragged_lengths(B, lo, hi, seed) -> np.ndarray:
    """B sequence lengths drawn uniformly from the integers lo..hi (seeded)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def _lengths(B, kv_lens, kv_len):
    """Per-sequence fill lengths: kv_lens if given, else kv_len for all."""
    if kv_lens is None:
        return np.full(B, kv_len, np.int32)
    lens = np.asarray(kv_lens, dtype=np.int32).reshape(-1)
    if lens.shape[0] != B:
        raise ValueError("kv_lens must hold one length per sequence")
    return lens


def gen_prefill(B, Hq, Hkv, N, D, dtype="bf16", seed=0, scale=None,
                outlier_frac=0.0, outlier_mult=8.0) -> Prefill:
    """Q, K, V i.i.d. N(0,1). With outlier_frac > 0, per (b, hkv) a seeded
    set of round(outlier_frac·N) distinct key rows is multiplied by
    outlier_mult after rounding (a power of two keeps that exact)."""
    rq, rk, rv, ro = _rng(seed, 4)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if dtype == "bf16":
        q = _normal_bf16(rq, (B, Hq, N, D))
        k = _normal_bf16(rk, (B, Hkv, N, D))
        v = _normal_bf16(rv, (B, Hkv, N, D))
    elif dtype == "f32":
        q = _normal(rq, (B, Hq, N, D))
        k = _normal(rk, (B, Hkv, N, D))
        v = _normal(rv, (B, Hkv, N, D))
    else:
        raise ValueError(dtype)
    rows = None
    n_out = int(round(outlier_frac * N))
    if n_out > 0:
        rows = np.stack([np.stack([np.sort(ro.choice(N, n_out, replace=False))
                                   for _ in range(Hkv)]) for _ in range(B)])
        for b in range(B):
            for h in range(Hkv):
                sel = rows[b, h]
                if dtype == "bf16":
                    k[b, h, sel] = round_to_bf16_bits(bf16_bits_as_f32(k[b, h, sel]) * outlier_mult)
                else:
                    k[b, h, sel] = k[b, h, sel] * np.float32(outlier_mult)
    return Prefill(B, Hq, Hkv, N, D, dtype, float(scale), q, k, v, rows)


def gen_upstream_grad(shape, seed) -> np.ndarray:
    """An upstream gradient dL/dO for the backward: N(0,1) draws in bf16."""
    return _normal_bf16(np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed))), shape)


def gen_decode_gqa(B, Hq, Hkv, kv_len=None, D=128, kv_cap=None, seed=0, scale=None,
                   poison_tail=True, kv_lens=None, cache_dtype="bf16") -> DecodeGQA:
    """One query token per sequence; K/V cache of capacity kv_cap filled to
    kv_len (or, for a ragged batch, sequence b filled to kv_lens[b]; kv_len
    is then the longest). Slots past a sequence's length hold NaN when
    poison_tail is set, so a kernel that reads them produces NaN. The cache
    holds bf16 or FP8 E4M3 (the same N(0,1) draws, rounded to that format);
    q is bf16 either way."""
    if kv_lens is not None:
        lens = _lengths(B, kv_lens, None)
        kv_len = int(lens.max())
    else:
        lens = _lengths(B, None, kv_len)
    if kv_cap is None:
        kv_cap = kv_len
    rq, rk, rv = _rng(seed, 3)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    q = _normal_bf16(rq, (B, Hq, D))
    if cache_dtype == "bf16":
        elt, draw, nan = np.uint16, _normal_bf16, BF16_NAN_BITS
    elif cache_dtype == "fp8":
        elt, draw, nan = np.uint8, _normal_e4m3, E4M3_NAN_BITS
    else:
        raise ValueError(cache_dtype)
    k = np.empty((B, Hkv, kv_cap, D), elt)
    v = np.empty((B, Hkv, kv_cap, D), elt)
    fill = nan if poison_tail else elt(0)
    for b in range(B):
        n = int(lens[b])
        k[b, :, :n] = draw(rk, (Hkv, n, D))
        v[b, :, :n] = draw(rv, (Hkv, n, D))
        k[b, :, n:] = fill
        v[b, :, n:] = fill
    return DecodeGQA(B, Hq, Hkv, kv_len, kv_cap, D, float(scale), q, k, v,
                     lens if kv_lens is not None else None, cache_dtype)


def gen_prefill_chunked(B, Hq, Hkv, Nq, kv_lens, D=128, kv_cap=None, seed=0, scale=None,
                        poison_tail=True) -> PrefillChunked:
    """A chunk of Nq query tokens per sequence against a cache filled to
    kv_lens[b] (a scalar applies to every sequence). All of Q and the filled
    K/V are N(0,1) in bf16; slots past a sequence's length hold NaN when
    poison_tail is set."""
    lens = _lengths(B, None, int(kv_lens)) if np.ndim(kv_lens) == 0 else _lengths(B, kv_lens, None)
    if lens.min() < Nq:
        raise ValueError("every sequence must hold at least the chunk's Nq tokens")
    if kv_cap is None:
        kv_cap = int(lens.max())
    rq, rk, rv = _rng(seed, 3)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    q = _normal_bf16(rq, (B, Hq, Nq, D))
    k = np.empty((B, Hkv, kv_cap, D), np.uint16)
    v = np.empty((B, Hkv, kv_cap, D), np.uint16)
    fill = BF16_NAN_BITS if poison_tail else np.uint16(0)
    for b in range(B):
        n = int(lens[b])
        k[b, :, :n] = _normal_bf16(rk, (Hkv, n, D))
        v[b, :, :n] = _normal_bf16(rv, (Hkv, n, D))
        k[b, :, n:] = fill
        v[b, :, n:] = fill
    return PrefillChunked(B, Hq, Hkv, Nq, kv_cap, D, float(scale), q, k, v, lens)


def gen_decode_mla(B, Hq, kv_len=None, Dqk=576, Dv=512, kv_cap=None, seed=0,
                   scale=None, mag_lo=1e-4, mag_hi=1e2, poison_tail=True,
                   kv_lens=None, cache_dtype="bf16", balance=True, calib_rows=128) -> DecodeMLA:
    """Absorbed-MLA decode inputs.

    Channel magnitudes: m_k = 10^U(log10 mag_lo, log10 mag_hi) per latent
    channel. The model-side absorbed query is q̃ = q_u ⊙ m and the latent is
    c = c_u ⊘ m (so logits stay O(1)), q_u, c_u ~ N(0,1). The rope channels
    (Dqk - Dv of them) are N(0,1) and not scaled.

    balance=True: a static channel scale S = diag(s) is applied before
    storage, q̃ ⊙ s⁻¹ and s ⊙ c. S is estimated offline, as the root mean
    square of each channel over `calib_rows` seeded calibration draws of that
    channel (magnitude m_k), so it tracks the true magnitudes only up to
    sampling error and some imbalance stays in storage. balance=False stores
    the raw q̃ and c (channels from mag_lo to mag_hi and their reciprocals).

    The default scale is 1/√192 (128 no-rope + 64 rope dims of the
    pre-absorption head). With kv_lens (a ragged batch) sequence b is filled
    to kv_lens[b] and kv_len is the longest. cache_dtype "fp8" stores the
    cache as OCP E4M3 codes of the same rows (round to nearest even; the
    balanced values lie far inside E4M3's range), the query staying bf16.
    """
    if cache_dtype not in ("bf16", "fp8"):
        raise ValueError(cache_dtype)
    fp8 = cache_dtype == "fp8"
    if kv_lens is not None:
        lens = _lengths(B, kv_lens, None)
        kv_len = int(lens.max())
    else:
        lens = _lengths(B, None, kv_len)
    if kv_cap is None:
        kv_cap = kv_len
    rq, rc, rs = _rng(seed, 3)
    if scale is None:
        scale = 1.0 / math.sqrt(128 + 64)
    mags = 10.0 ** rs.uniform(math.log10(mag_lo), math.log10(mag_hi), size=Dv)
    if balance:
        calib = rs.standard_normal((calib_rows, Dv)) * mags
        s = np.sqrt(np.mean(calib * calib, axis=0))
    else:
        s = np.ones(Dv)
    qn = _normal(rq, (B, Hq, Dqk)).astype(np.float64)
    q_tilde = qn[..., :Dv] * mags                   # raw absorbed query
    qn[..., :Dv] = q_tilde / s                      # q̃·S⁻¹
    q = round_to_bf16_bits(qn)
    elt, nan = (np.uint8, E4M3_NAN_BITS) if fp8 else (np.uint16, BF16_NAN_BITS)
    ckv = np.empty((B, kv_cap, Dqk), elt)
    for b in range(B):                              # per batch to bound memory
        n = int(lens[b])
        cn = _normal(rc, (n, Dqk)).astype(np.float64)
        c_raw = cn[:, :Dv] / mags                   # raw latent
        cn[:, :Dv] = s * c_raw                      # S·c
        ckv[b, :n] = round_to_e4m3_bits(cn) if fp8 else round_to_bf16_bits(cn)
        ckv[b, n:] = nan if poison_tail else elt(0)
    return DecodeMLA(B, Hq, kv_len, kv_cap, Dqk, Dv, float(scale), q, ckv, s,
                     lens if kv_lens is not None else None, cache_dtype, mags)


# --------------------------------------------------------- named workloads ---
WORKLOADS = {
    "prefill_f32_tiny": dict(
        kind="prefill", B=1, Hq=2, Hkv=2, N=64, D=64, dtype="f32", seed=1001,
        scale=1.0 / 8.0),
    "decode_gqa_llama3_8b_4k": dict(
        kind="decode_gqa", B=8, Hq=32, Hkv=8, kv_len=4096, D=128, seed=1002,
        scale=1.0 / math.sqrt(128)),
    "prefill_bf16_4k": dict(
        kind="prefill", B=4, Hq=32, Hkv=8, N=4096, D=128, dtype="bf16", seed=1003,
        scale=1.0 / math.sqrt(128)),
    "prefill_bf16_32k_outliers": dict(
        kind="prefill", B=1, Hq=32, Hkv=8, N=32768, D=128, dtype="bf16", seed=1004,
        scale=1.0 / math.sqrt(128), outlier_frac=0.01, outlier_mult=8.0),
    "decode_mla_absorbed_32k": dict(
        kind="decode_mla", B=16, Hq=128, kv_len=32768, Dqk=576, Dv=512, seed=1005,
        scale=1.0 / math.sqrt(128 + 64)),
    # serving shapes of the same kernels: a prompt chunk appended to a cache
    # (bottom-right causal mask) and decode batches of mixed lengths
    "prefill_chunked_4k_on_32k": dict(
        kind="prefill_chunked", B=1, Hq=32, Hkv=8, Nq=4096, kv_lens=32768, D=128,
        seed=1006, scale=1.0 / math.sqrt(128)),
    "prefill_chunked_512_on_32k": dict(
        kind="prefill_chunked", B=1, Hq=32, Hkv=8, Nq=512, kv_lens=32768, D=128,
        seed=1011, scale=1.0 / math.sqrt(128)),
    "decode_gqa_ragged_8k": dict(
        kind="decode_gqa", B=32, Hq=32, Hkv=8, kv_lens=("ragged", 128, 8192, 1107),
        kv_cap=8192, D=128, seed=1007, scale=1.0 / math.sqrt(128)),
    # the backward of the 4k prefill (upstream gradient seed 1010)
    "prefill_bf16_4k_backward": dict(
        kind="prefill_backward", B=4, Hq=32, Hkv=8, N=4096, D=128, dtype="bf16", seed=1003,
        scale=1.0 / math.sqrt(128)),
    # the Llama-3-8B decode with an FP8 E4M3 K/V cache (half the bytes)
    "decode_gqa_fp8_llama3_8b_4k": dict(
        kind="decode_gqa", B=8, Hq=32, Hkv=8, kv_len=4096, D=128, seed=1009,
        scale=1.0 / math.sqrt(128), cache_dtype="fp8"),
    "decode_mla_fp8_32k": dict(
        kind="decode_mla", B=16, Hq=128, kv_len=32768, Dqk=576, Dv=512, seed=1010,
        scale=1.0 / math.sqrt(128 + 64), cache_dtype="fp8"),
    "decode_mla_ragged_32k": dict(
        kind="decode_mla", B=16, Hq=128, kv_lens=("ragged", 1024, 32768, 1108),
        kv_cap=32768, Dqk=576, Dv=512, seed=1008, scale=1.0 / math.sqrt(128 + 64)),
    # the same ragged batch over an E4M3 latent cache
    "decode_mla_ragged_fp8_32k": dict(
        kind="decode_mla", B=16, Hq=128, kv_lens=("ragged", 1024, 32768, 1108),
        kv_cap=32768, Dqk=576, Dv=512, seed=1008, scale=1.0 / math.sqrt(128 + 64),
        cache_dtype="fp8"),
}


def make(name: str, **overrides):
    """Build a named workload (overrides change shapes for scaled-down cases)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    lens = cfg.get("kv_lens")
    if isinstance(lens, tuple) and lens and lens[0] == "ragged":
        cfg["kv_lens"] = ragged_lengths(cfg["B"], *lens[1:])
    if kind == "prefill_chunked":
        return gen_prefill_chunked(**cfg)
    if kind == "prefill_backward":
        return gen_prefill(**cfg)
    if kind == "prefill":
        return gen_prefill(**cfg)
    if kind == "decode_gqa":
        return gen_decode_gqa(**cfg)
    if kind == "decode_mla":
        return gen_decode_mla(**cfg)
    raise ValueError(kind)


# ------------------------------------------ algorithmic work per launch ---
def prefill_causal_flops(B, Hq, N, D):
    """Flops of the unmasked (i, j≤i) pairs only: 2·D for q·k plus 2·D for
    p·v per pair. Skipped tiles and masked diagonal entries are not counted."""
    return 4 * D * (N * (N + 1) // 2) * B * Hq


def prefill_min_bytes(B, Hq, Hkv, N, D, elt=2):
    """Compulsory HBM bytes: Q, K, V read once, O written once, fp32 LSE."""
    return elt * N * D * (2 * B * Hq + 2 * B * Hkv) + 4 * B * Hq * N


def decode_gqa_bytes(B, Hq, Hkv, kv_len, D, elt=2, kv_elt=None):
    """K and V rows up to kv_len read once (kv_elt bytes per element, 1 for
    an FP8 cache), q read, O written (elt bytes), fp32 LSE."""
    kv_elt = elt if kv_elt is None else kv_elt
    return kv_elt * 2 * B * Hkv * kv_len * D + elt * 2 * B * Hq * D + 4 * B * Hq


def decode_gqa_flops(B, Hq, kv_len, D):
    return 4 * B * Hq * kv_len * D


def decode_mla_bytes(B, Hq, kv_len, Dqk, Dv, elt=2, kv_elt=None):
    """Latent rows read once (V is a prefix of each row; kv_elt bytes per
    element, 1 for an FP8 cache), q, O (elt bytes), fp32 LSE."""
    kv_elt = elt if kv_elt is None else kv_elt
    return kv_elt * B * kv_len * Dqk + elt * (B * Hq * Dqk + B * Hq * Dv) + 4 * B * Hq


def decode_mla_flops(B, Hq, kv_len, Dqk, Dv):
    return 2 * B * Hq * kv_len * (Dqk + Dv)


def prefill_chunked_flops(Hq, Nq, kv_lens, D):
    """Flops of the visible pairs of a chunk against its cache: chunk row i
    of sequence b sees kv_lens[b] − Nq + i + 1 keys; 4·D flops per pair."""
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(-1)
    pairs = int(np.sum(Nq * (lens - Nq) + Nq * (Nq + 1) // 2))
    return 4 * D * pairs * Hq


def decode_gqa_ragged_bytes(Hq, Hkv, kv_lens, D, elt=2):
    """As decode_gqa_bytes with per-sequence filled lengths."""
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(-1)
    B = lens.shape[0]
    return int(elt * (2 * Hkv * int(lens.sum()) * D + 2 * B * Hq * D) + 4 * B * Hq)


def decode_mla_ragged_bytes(Hq, kv_lens, Dqk, Dv, kv_elt=2):
    """As decode_mla_bytes with per-sequence filled lengths (kv_elt bytes per
    cached element: 2 for bf16, 1 for E4M3; q and O are bf16)."""
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(-1)
    B = lens.shape[0]
    return int(kv_elt * int(lens.sum()) * Dqk + 2 * (B * Hq * Dqk + B * Hq * Dv) + 4 * B * Hq)


def prefill_backward_flops(B, Hq, N, D):
    """Algorithmic flops of the backward over the visible pairs: the five
    products of the standard recomputing backward (S, dP, dV, dQ, dK), 2·D
    flops each per pair. (The kernels here form S and dP twice, once for
    dK/dV and once for dQ; that extra work is not counted.)"""
    return 10 * D * (N * (N + 1) // 2) * B * Hq
