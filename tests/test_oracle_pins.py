"""Pins for the fp64 oracle: each test checks the oracle against something
other than itself — values the pages print, closed forms, brute force on tiny
hand-worked inputs, or an independent library routine (torch's CPU float64
scaled_dot_product_attention / logsumexp).

Pages are cited by title and section; the printed values live in
tests/golden/page_examples.json next to their citations.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def _decode_1q(q_vec, keys, values=None, scale=1.0):
    """Helper: one query (B=Hq=Hkv=1) against explicit keys/values."""
    q = np.asarray(q_vec, dtype=np.float64)[None, None, :]
    k = np.asarray(keys, dtype=np.float64)[None, None, :, :]
    v = k.copy() if values is None else np.asarray(values, dtype=np.float64)[None, None, :, :]
    o, lse, p = oracle.decode_gqa(q, k, v, k.shape[2], scale, return_p=True)
    return o[0, 0], lse[0, 0], p[0, 0]


# ------------------------------------------------------- page-printed values ---
def test_dot_product_page_value():
    """05 · Tích vô hướng…, §1: (2,−1,0.5)·(3,4,2) = 3. One visible key:
    its weight is 1, so LSE equals the (unscaled) score exactly."""
    g = GOLD["dot_product"]
    o, lse, p = _decode_1q(g["a"], [g["b"]], scale=1.0)
    assert lse == g["expected"]
    assert p[0] == 1.0
    np.testing.assert_array_equal(o, g["b"])


def test_softmax_page_values():
    """05 · Tích vô hướng…, §2: scores 2, 1, 0.1 → e^x ≈ 7.39, 2.72, 1.11,
    sum ≈ 11.2, weights ≈ 66 %, 24 %, 10 %."""
    g = GOLD["softmax_three_scores"]
    _, lse, p = _decode_1q([1.0], [[s] for s in g["scores"]])
    np.testing.assert_allclose(p, g["weights"], atol=g["weights_tol"])
    assert abs(math.exp(lse) - g["exp_sum"]) < g["exp_sum_tol"]
    np.testing.assert_allclose(p * math.exp(lse), g["exp_values"], atol=g["exp_values_tol"])
    assert abs(p.sum() - 1.0) < 1e-15


def test_safe_softmax_shift_page_and_overflow():
    """05 · Tích vô hướng…, §2 and Bộ 06 Q1: subtracting the row max (2, 1,
    0.1 → 0, −1, −1.9) leaves the weights unchanged; softmax(x−c) =
    softmax(x) even where an unshifted e^x would overflow."""
    g = GOLD["safe_softmax_shift"]
    _, _, p_ref = _decode_1q([1.0], [[s] for s in g["scores"]])
    _, _, p_sh = _decode_1q([1.0], [[s] for s in g["shifted"]])
    np.testing.assert_allclose(p_sh, p_ref, rtol=0, atol=1e-15)
    assert abs(math.exp(12) - g["exp12"]) < g["exp12_tol"] and math.exp(12) > g["fp16_max"]
    for c in (1000.0, -1000.0):
        _, lse, p = _decode_1q([1.0], [[s + c] for s in g["scores"]])
        assert np.all(np.isfinite(p)) and math.isfinite(lse)
        np.testing.assert_allclose(p, p_ref, rtol=0, atol=1e-13)


def _online_blocks(blocks):
    """Test-only online softmax over blocks of scores: running max m and
    running sum ℓ, old sum rescaled by e^(m_old − m_new) when m grows
    (05 · Tích vô hướng…, §6; Bộ 06, Q1 follow-up)."""
    m, l, ms = -math.inf, 0.0, []
    for blk in blocks:
        m_new = max(m, max(blk))
        l = l * math.exp(m - m_new) + sum(math.exp(s - m_new) for s in blk)
        m = m_new
        ms.append(m)
    return m, l, ms


def test_online_blocks_page_value():
    """05 · Tích vô hướng…, §6: blocks [2, 1] then [3, 0] give a running sum
    ≈ 1.55, equal to the whole-row result; the running max never falls."""
    g = GOLD["online_softmax_blocks"]
    m_on, l_on, ms = _online_blocks(g["blocks"])
    assert abs(l_on - g["running_sum"]) < g["running_sum_tol"]
    assert ms == sorted(ms)
    flat = [s for blk in g["blocks"] for s in blk]
    _, lse, _ = _decode_1q([1.0], [[s] for s in flat])
    m_full = max(flat)
    l_full = math.exp(lse - m_full)
    assert m_on == m_full
    assert abs(l_full - g["running_sum"]) < g["running_sum_tol"]
    assert abs(l_full - l_on) < 1e-14


def test_causal_mask_pattern_page_picture():
    """第11节 §3: the 4×4 triu(1) picture — row i sees keys 0..i; masked
    entries get exactly zero weight (Bộ 06 Q2: e^(−∞) = 0)."""
    vis = np.array(GOLD["causal_mask_4x4"]["visible"], dtype=bool)
    w = workloads.gen_prefill(1, 1, 1, 4, 8, dtype="f32", seed=7)
    _, _, p = oracle.prefill_causal(w.q, w.k, w.v, w.scale, return_p=True)
    p = p[0, 0]
    assert np.all(p[~vis] == 0.0)
    assert np.all(p[vis] > 0.0)


def test_kv_recompute_count_page_values():
    """Bộ 06 Q2: naive recompute = N·P + N(N−1)/2 = 131,072 + 32,640 ≈ 164k
    token passes versus P + N = 768 cached, ≈ 213× waste. Counted by
    running the two loops' bookkeeping, not by the formula."""
    g = GOLD["kv_cache_recompute_count"]
    P, N = g["prompt_tokens"], g["generated_tokens"]
    naive = sum(P + n for n in range(N))          # step n re-feeds P + n tokens
    cached = P + sum(1 for _ in range(N))         # prompt once, then one per token
    assert naive == sum(g["naive_terms"])
    assert abs(naive - g["naive_total_approx"]) < 500
    assert cached == g["cached_total"]
    assert round(naive / cached) == g["waste_ratio_approx"]


def test_llama_decode_bill_page_values():
    """05 · Tích vô hướng…, §4 and Bộ 06 Q2: per decoded token at 4096
    context, 4,194,304 dots ≈ 2.1 B ops against ≈ 0.5 GB of K/V
    (4 KiB/token/layer, 128 KiB/token), ≈ 4 ops/byte. Pins the counters
    the bench prices launches with."""
    g = GOLD["llama3_8b_decode_bill"]
    L, Hq, Hkv, T, D = g["layers"], g["q_heads"], g["kv_heads"], g["context"], g["head_dim"]
    assert L * Hq * T == g["dots"]
    ops = L * workloads.decode_gqa_flops(1, Hq, T, D)
    assert abs(ops - g["ops_approx"]) < g["ops_tol"]
    extra = workloads.decode_gqa_bytes(1, Hq, Hkv, 0, D)   # q, O, LSE only
    kv_per_token_layer = workloads.decode_gqa_bytes(1, Hq, Hkv, 1, D) - extra
    assert kv_per_token_layer == g["kv_bytes_per_token_layer"]
    assert L * kv_per_token_layer == g["kv_bytes_per_token"]
    kv_ctx = L * (workloads.decode_gqa_bytes(1, Hq, Hkv, T, D) - extra)
    assert abs(kv_ctx - g["kv_bytes_context_approx"]) < g["kv_bytes_tol"]
    assert round(ops / kv_ctx) == g["ops_per_byte_approx"]


def test_generator_score_spread_page_value():
    """05 · Tích vô hướng…, §1 and Bộ 06 Q1: unit-variance d=128 vectors give
    dot products with spread √128 ≈ 11.3; ÷√128 brings it back to ≈ 1."""
    g = GOLD["score_spread_d128"]
    w = workloads.gen_prefill(1, 1, 1, 2048, g["head_dim"], dtype="bf16", seed=3)
    q = workloads.bf16_bits_as_f32(w.q[0, 0]).astype(np.float64)
    k = workloads.bf16_bits_as_f32(w.k[0, 0]).astype(np.float64)
    s = np.einsum("id,id->i", q, k)
    assert abs(s.std() - g["raw_spread"]) / g["raw_spread"] < 0.05
    assert abs(s.std() * w.scale - g["scaled_spread"]) < 0.05


# ------------------------------------------------------------- closed forms ---
def test_hand_worked_two_tokens():
    """Brute force by hand: Q=[[0],[1]], K=[[1],[2]], V=[[0],[1]], scale 1.
    Row 0 sees only key 0: O=0, LSE=0·1=0. Row 1 scores (1, 2):
    O = e²/(e+e²) = e/(1+e), LSE = ln(e + e²) = 1 + ln(1+e)."""
    q = np.array([[[[0.0], [1.0]]]])
    k = np.array([[[[1.0], [2.0]]]])
    v = np.array([[[[0.0], [1.0]]]])
    o, lse = oracle.prefill_causal(q, k, v, 1.0)
    e = math.e
    assert o[0, 0, 0, 0] == 0.0 and lse[0, 0, 0] == 0.0
    assert abs(o[0, 0, 1, 0] - e / (1 + e)) < 1e-15
    assert abs(lse[0, 0, 1] - (1 + math.log(1 + e))) < 1e-15


def test_hand_worked_three_tokens_integer():
    """Brute force: D=2, scale 1/2, Q rows (2,0), (0,2), (2,2); K rows
    (1,0), (0,1), (1,1); V rows (1,0), (0,1), (3,3).
    Row 0: one key → O=V0, LSE = ½·2 = 1.
    Row 1: scores (0, 1) → weights 1/(1+e), e/(1+e).
    Row 2: scores (1, 1, 2) → weights (1, 1, e)/(2+e), LSE = 1 + ln(2+e)."""
    q = np.array([[[[2, 0], [0, 2], [2, 2]]]], dtype=np.float64)
    k = np.array([[[[1, 0], [0, 1], [1, 1]]]], dtype=np.float64)
    v = np.array([[[[1, 0], [0, 1], [3, 3]]]], dtype=np.float64)
    o, lse, p = oracle.prefill_causal(q, k, v, 0.5, return_p=True)
    e = math.e
    np.testing.assert_array_equal(o[0, 0, 0], [1.0, 0.0])
    assert lse[0, 0, 0] == 1.0
    np.testing.assert_allclose(p[0, 0, 1], [1 / (1 + e), e / (1 + e), 0.0], rtol=0, atol=1e-16)
    np.testing.assert_allclose(o[0, 0, 1], [1 / (1 + e), e / (1 + e)], rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 1] - math.log(1 + e)) < 1e-15
    w2 = np.array([1, 1, e]) / (2 + e)
    np.testing.assert_allclose(p[0, 0, 2], w2, rtol=0, atol=1e-16)
    np.testing.assert_allclose(o[0, 0, 2], [w2[0] + 3 * w2[2], w2[1] + 3 * w2[2]], rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 2] - (1 + math.log(2 + e))) < 1e-15


def test_zero_query_uniform_weights():
    """Q = 0 makes every visible score 0, so the weights are uniform:
    O[i] = mean(V[0..i]) and LSE[i] = ln(i+1)."""
    w = workloads.gen_prefill(2, 4, 2, 33, 16, dtype="f32", seed=11)
    q = np.zeros_like(w.q)
    o, lse = oracle.prefill_causal(q, w.k, w.v, w.scale)
    v = w.v.astype(np.float64)
    for hq in range(4):
        hkv = hq // 2
        cm = np.cumsum(v[:, hkv], axis=1) / np.arange(1, 34)[None, :, None]
        np.testing.assert_allclose(o[:, hq], cm, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, hq], np.broadcast_to(np.log(np.arange(1, 34)), (2, 33)),
                                   rtol=0, atol=1e-14)


def test_row0_equals_v0_and_lse_is_score():
    """第11节 §3: query 0 sees only key 0, so O[0] = V[0] exactly and
    LSE[0] = scale·q0·k0."""
    w = workloads.gen_prefill(2, 8, 2, 40, 64, dtype="bf16", seed=5)
    o, lse = oracle.prefill_causal(w.q, w.k, w.v, w.scale, rows=[0, 1, 39])
    q, k, v = oracle.widen(w.q), oracle.widen(w.k), oracle.widen(w.v)
    for hq in range(8):
        hkv = hq // 4
        np.testing.assert_array_equal(o[:, hq, 0], v[:, hkv, 0])
        s00 = w.scale * np.einsum("bd,bd->b", q[:, hq, 0], k[:, hkv, 0])
        np.testing.assert_allclose(lse[:, hq, 0], s00, rtol=1e-14, atol=1e-15)


def test_rows_sum_to_one():
    w = workloads.gen_prefill(1, 2, 1, 50, 32, dtype="f32", seed=9)
    _, _, p = oracle.prefill_causal(w.q, w.k, w.v, w.scale, return_p=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)


# ------------------------------------------------- library special cases ---
def _torch_sdpa(q, k, v, scale, causal):
    import torch
    import torch.nn.functional as F
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    return F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale,
                                          enable_gqa=True).numpy()


def _torch_lse(q, k, scale, causal):
    import torch
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    s = (qt @ kt.transpose(-1, -2)) * scale
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    return torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("B,Hq,Hkv,N,D", [(2, 4, 2, 37, 16), (1, 8, 1, 70, 64), (1, 3, 3, 5, 8)])
def test_prefill_matches_torch_sdpa(B, Hq, Hkv, N, D):
    """Library special case: torch's CPU float64 SDPA with is_causal and
    contiguous GQA groups (enable_gqa repeats each K/V head for Hq/Hkv
    consecutive query heads) computes the same O; torch.logsumexp over the
    masked scores gives the same LSE."""
    w = workloads.gen_prefill(B, Hq, Hkv, N, D, dtype="bf16", seed=21)
    q, k, v = oracle.widen(w.q), oracle.widen(w.k), oracle.widen(w.v)
    o, lse = oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    np.testing.assert_allclose(o, _torch_sdpa(q, k, v, w.scale, True), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _torch_lse(q, k, w.scale, True), rtol=0, atol=1e-12)


def test_decode_matches_torch_sdpa_and_ignores_unfilled_slots():
    """Decode (no mask) against torch SDPA on the filled prefix; slots past
    kv_len hold NaN and must not reach the result (Bộ 06 Q3)."""
    w = workloads.gen_decode_gqa(3, 8, 2, 45, D=32, kv_cap=64, seed=4, poison_tail=True)
    o, lse = oracle.decode_gqa(w.q, w.k, w.v, w.kv_len, w.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    q = oracle.widen(w.q)[:, :, None, :]
    k = oracle.widen(w.k[:, :, :w.kv_len])
    v = oracle.widen(w.v[:, :, :w.kv_len])
    np.testing.assert_allclose(o, _torch_sdpa(q, k, v, w.scale, False)[:, :, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _torch_lse(q, k, w.scale, False)[:, :, 0], rtol=0, atol=1e-12)


def test_mla_matches_torch_sdpa():
    """MLA absorbed decode = multi-query attention with one latent head:
    key = the whole 576-wide row, value = its first 512 channels. torch SDPA
    with a shared K/V head (expand) and a narrower V computes the same."""
    import torch
    import torch.nn.functional as F
    w = workloads.gen_decode_mla(2, 16, 300, Dqk=72, Dv=64, kv_cap=320, seed=8)
    o, lse = oracle.decode_mla_absorbed(w.q, w.ckv, w.kv_len, w.Dv, w.scale)
    q = torch.from_numpy(oracle.widen(w.q))[:, :, None, :]
    c = torch.from_numpy(oracle.widen(w.ckv[:, :w.kv_len]))[:, None]
    k = c.expand(-1, 16, -1, -1)
    v = c[..., :w.Dv].expand(-1, 16, -1, -1)
    ref = F.scaled_dot_product_attention(q, k, v, scale=w.scale)[:, :, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    s = (q @ k.transpose(-1, -2))[:, :, 0] * w.scale
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


def test_mla_channel_balance_is_exact_in_real_arithmetic():
    """MLA 矩阵乘法吸收… §二.1: (q̃S⁻¹)·(Sc) = q̃·c, so attending with the
    balanced pair gives the same LSE, and O in the balanced space is S·O_raw."""
    rng = np.random.default_rng(2)
    B, Hq, L, Dv, R = 1, 4, 50, 32, 8
    s = 10.0 ** rng.uniform(-4, 2, size=Dv)
    q_tilde = np.concatenate([rng.standard_normal((B, Hq, Dv)) * s, rng.standard_normal((B, Hq, R))], -1)
    c_raw = np.concatenate([rng.standard_normal((B, L, Dv)) / s, rng.standard_normal((B, L, R))], -1)
    q_bal = q_tilde.copy(); q_bal[..., :Dv] /= s
    c_bal = c_raw.copy(); c_bal[..., :Dv] *= s
    o_raw, lse_raw = oracle.decode_mla_absorbed(q_tilde, c_raw, L, Dv, 0.2)
    o_bal, lse_bal = oracle.decode_mla_absorbed(q_bal, c_bal, L, Dv, 0.2)
    np.testing.assert_allclose(lse_bal, lse_raw, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o_bal / s, o_raw, rtol=1e-9, atol=1e-12)


# ------------------------------------------------------------- invariants ---
def test_kv_cache_rows_match_prefill_bitwise():
    """Bộ 06 Q2/Q3: a new token lies in every earlier row's masked future, so
    decoding token t against the cached K/V[0..t] equals prefill row t —
    exactly (the masked keys add exact zeros)."""
    w = workloads.gen_prefill(1, 4, 2, 24, 16, dtype="bf16", seed=13)
    o_p, lse_p = oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    for t in range(24):
        o_d, lse_d = oracle.decode_gqa(w.q[:, :, t], w.k[:, :, :t + 1], w.v[:, :, :t + 1], t + 1, w.scale)
        np.testing.assert_array_equal(o_d, o_p[:, :, t])
        np.testing.assert_array_equal(lse_d, lse_p[:, :, t])


def test_thread_count_does_not_change_results():
    w = workloads.gen_prefill(1, 4, 2, 60, 32, dtype="bf16", seed=17)
    a = oracle.prefill_causal(w.q, w.k, w.v, w.scale, threads=1)
    b = oracle.prefill_causal(w.q, w.k, w.v, w.scale, threads=5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_row_subset_equals_full():
    w = workloads.gen_prefill(1, 2, 1, 48, 16, dtype="f32", seed=19)
    o, lse = oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    rows = [47, 0, 13]
    o_s, lse_s = oracle.prefill_causal(w.q, w.k, w.v, w.scale, rows=rows)
    np.testing.assert_array_equal(o_s, o[:, :, rows])
    np.testing.assert_array_equal(lse_s, lse[:, :, rows])


def test_oracle_rejects_bad_arguments():
    w = workloads.gen_prefill(1, 3, 2, 8, 8, dtype="f32", seed=1)   # Hq % Hkv != 0
    with pytest.raises(ValueError):
        oracle.prefill_causal(w.q, w.k, w.v, w.scale)
    with pytest.raises(ValueError):
        oracle.prefill_causal(w.q[:, :2], w.k, w.v, w.scale, rows=[8])


# ------------------------------------------ chunked prefill and ragged decode ---
def test_chunked_mask_page_picture():
    """第11节 §3: with K = [history | chunk], the triu(1) mask covers only the
    chunk's own columns. With one-hot values (V[j] = e_j) the output row is
    the weight row itself: every history key and chunk keys 0..i carry
    weight > 0; chunk keys after i carry exactly 0 (the 4×4 picture)."""
    vis4 = np.array(GOLD["causal_mask_4x4"]["visible"], dtype=bool)
    past, Nq = 3, 4
    L = past + Nq
    w = workloads.gen_prefill_chunked(1, 2, 1, Nq, L, D=L, seed=31)
    eye = workloads.round_to_bf16_bits(np.eye(L, dtype=np.float32))
    v = eye[None, None]
    o, _ = oracle.prefill_chunked(w.q, w.k, v, w.kv_lens, w.scale)
    for hq in range(2):
        p = o[0, hq]                                  # [Nq, L] weights
        assert np.all(p[:, :past] > 0.0)
        assert np.all(p[:, past:][~vis4] == 0.0)
        assert np.all(p[:, past:][vis4] > 0.0)
        np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)


def test_chunked_rows_equal_full_prefill_bitwise():
    """Bộ 06 Q2 (cached K/V are exact) with 第11节 §3: the chunk's rows are the
    last Nq rows of a causal prefill over history + chunk, bit for bit (the
    same scores in the same order; masked keys add exact zeros)."""
    Nq, L = 9, 30
    w = workloads.gen_prefill_chunked(2, 4, 2, Nq, L, D=16, seed=32)
    o_c, lse_c = oracle.prefill_chunked(w.q, w.k, w.v, w.kv_lens, w.scale)
    full_q = np.zeros((2, 4, L, 16), np.uint16)
    full_q[:, :, L - Nq:] = w.q
    o_f, lse_f = oracle.prefill_causal(full_q, w.k[:, :, :L], w.v[:, :, :L], w.scale,
                                       rows=np.arange(L - Nq, L))
    np.testing.assert_array_equal(o_c, o_f)
    np.testing.assert_array_equal(lse_c, lse_f)


def test_chunked_matches_torch_sdpa_on_the_full_sequence():
    """Library special case: torch's CPU float64 SDPA with is_causal over the
    whole sequence (history + chunk), last Nq rows; ragged lengths per
    sequence, contiguous GQA groups."""
    Nq, lens = 7, [7, 19, 40]
    w = workloads.gen_prefill_chunked(3, 6, 2, Nq, lens, D=32, kv_cap=44, seed=33)
    o, lse = oracle.prefill_chunked(w.q, w.k, w.v, w.kv_lens, w.scale)
    for b, L in enumerate(lens):
        k = oracle.widen(w.k[b:b + 1, :, :L])
        v = oracle.widen(w.v[b:b + 1, :, :L])
        q = np.zeros((1, 6, L, 32))
        q[:, :, L - Nq:] = oracle.widen(w.q[b:b + 1])
        ref = _torch_sdpa(q, k, v, w.scale, True)[:, :, L - Nq:]
        np.testing.assert_allclose(o[b:b + 1], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b:b + 1], _torch_lse(q, k, w.scale, True)[:, :, L - Nq:],
                                   rtol=0, atol=1e-12)


def test_chunked_zero_query_uniform_weights():
    """Q = 0: chunk row i sees P + i + 1 keys with equal weights, so
    O[i] = mean(V[0..P+i]) and LSE[i] = ln(P + i + 1)."""
    Nq, L = 6, 25
    w = workloads.gen_prefill_chunked(1, 2, 1, Nq, L, D=8, seed=34)
    q = np.zeros_like(w.q)
    o, lse = oracle.prefill_chunked(q, w.k, w.v, w.kv_lens, w.scale)
    v = oracle.widen(w.v[0, 0, :L])
    P = L - Nq
    for i in range(Nq):
        np.testing.assert_allclose(o[0, :, i], np.broadcast_to(v[:P + i + 1].mean(0), (2, 8)),
                                   rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], math.log(P + i + 1), rtol=0, atol=1e-14)


def test_chunk_of_one_token_is_decode():
    """A one-token chunk is a decode step: no chunk key lies after it, so it
    sees the whole filled cache (Bộ 06 Q2) — bit for bit the decode result."""
    w = workloads.gen_prefill_chunked(2, 4, 2, 1, [5, 33], D=16, kv_cap=40, seed=35)
    o, lse = oracle.prefill_chunked(w.q, w.k, w.v, w.kv_lens, w.scale)
    for b, L in enumerate(w.kv_lens):
        o_d, lse_d = oracle.decode_gqa(w.q[b:b + 1, :, 0], w.k[b:b + 1], w.v[b:b + 1], int(L), w.scale)
        np.testing.assert_array_equal(o[b:b + 1, :, 0], o_d)
        np.testing.assert_array_equal(lse[b:b + 1, :, 0], lse_d)


def test_ragged_decode_is_per_sequence_decode():
    """A ragged batch is B independent decodes, each over its own filled
    prefix (Bộ 06 Q3): bit for bit, for GQA and for absorbed MLA; the NaN
    tail past each length never reaches the result."""
    lens = [1, 17, 64, 40]
    w = workloads.gen_decode_gqa(4, 8, 2, D=32, kv_cap=64, kv_lens=lens, seed=36)
    o, lse = oracle.decode_gqa_ragged(w.q, w.k, w.v, w.kv_lens, w.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b, L in enumerate(lens):
        o_d, lse_d = oracle.decode_gqa(w.q[b:b + 1], w.k[b:b + 1], w.v[b:b + 1], L, w.scale)
        np.testing.assert_array_equal(o[b:b + 1], o_d)
        np.testing.assert_array_equal(lse[b:b + 1], lse_d)
    m = workloads.gen_decode_mla(3, 16, Dqk=72, Dv=64, kv_cap=50, kv_lens=[50, 3, 21], seed=37)
    o, lse = oracle.decode_mla_ragged(m.q, m.ckv, m.kv_lens, m.Dv, m.scale)
    for b, L in enumerate(m.kv_lens):
        o_d, lse_d = oracle.decode_mla_absorbed(m.q[b:b + 1], m.ckv[b:b + 1], int(L), m.Dv, m.scale)
        np.testing.assert_array_equal(o[b:b + 1], o_d)
        np.testing.assert_array_equal(lse[b:b + 1], lse_d)


def test_ragged_decode_zero_query_and_empty_sequence():
    """Q = 0: O = mean(V[:L]), LSE = ln L. A sequence with no filled slot has
    empty sums: O = 0 and LSE = ln 0 = −∞ (no NaN)."""
    lens = [0, 1, 9]
    w = workloads.gen_decode_gqa(3, 4, 2, D=16, kv_cap=12, kv_lens=lens, seed=38)
    o, lse = oracle.decode_gqa_ragged(np.zeros_like(w.q), w.k, w.v, w.kv_lens, w.scale)
    assert np.all(o[0] == 0.0) and np.all(lse[0] == -np.inf)
    for b in (1, 2):
        v = oracle.widen(w.v[b, :, :lens[b]])            # [Hkv, L, D]
        np.testing.assert_allclose(o[b], np.repeat(v.mean(1), 2, axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], math.log(lens[b]), rtol=0, atol=1e-15)
    m = workloads.gen_decode_mla(2, 16, Dqk=24, Dv=16, kv_cap=8, kv_lens=[0, 8], seed=39)
    o, lse = oracle.decode_mla_ragged(m.q, m.ckv, m.kv_lens, m.Dv, m.scale)
    assert np.all(o[0] == 0.0) and np.all(lse[0] == -np.inf) and np.all(np.isfinite(o[1]))


def test_chunked_and_ragged_reject_bad_lengths():
    w = workloads.gen_prefill_chunked(1, 2, 1, 4, 10, D=8, seed=40)
    with pytest.raises(ValueError):       # shorter than the chunk
        oracle.prefill_chunked(w.q, w.k, w.v, [3], w.scale)
    with pytest.raises(ValueError):       # one length per sequence
        oracle.prefill_chunked(w.q, w.k, w.v, [10, 10], w.scale)
    d = workloads.gen_decode_gqa(2, 2, 1, D=8, kv_cap=6, kv_lens=[2, 6], seed=41)
    with pytest.raises(ValueError):
        oracle.decode_gqa_ragged(d.q, d.k, d.v, [-1, 3], d.scale)


def test_e4m3_widening_matches_the_format_definition():
    """OCP FP8 E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
    subnormals m·2^-9, no infinity, S.1111.111 = NaN, largest finite 448.
    Spot values of the definition, and the grid between them: from a code
    of exponent e the next code is 2^(e−10) higher, and the subnormals
    continue the first binade's spacing down to 0."""
    c = np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0x80, 0xB8, 0xFE], np.uint8)
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 448.0, -0.0, -1.0, -448.0]
    got = oracle.widen(c)
    np.testing.assert_array_equal(got, want)
    assert np.signbit(got[7]) and not np.signbit(got[0])
    assert np.all(np.isnan(oracle.widen(np.array([0x7F, 0xFF], np.uint8))))
    pos = oracle.widen(np.arange(0x7F, dtype=np.uint8))
    steps = np.diff(pos)
    for code in range(1, 0x7F):
        e = max((code - 1) >> 3, 1)   # the spacing of the lower code's binade
        assert steps[code - 1] == 2.0 ** (e - 10), code
    np.testing.assert_array_equal(oracle.widen(np.arange(0x80, 0xFF, dtype=np.uint8)), -pos)


def test_decode_over_fp8_cache_is_decode_over_its_values():
    """An FP8 cache is attended to through its exact values: the decode of
    E4M3 K/V equals the decode of the same values held in float64, bit for
    bit, and the NaN tail past kv_len is never read."""
    w = workloads.gen_decode_gqa(2, 8, 2, 40, D=16, kv_cap=48, seed=5, cache_dtype="fp8")
    assert w.k.dtype == np.uint8 and np.isnan(oracle.widen(w.k[:, :, 40:])).all()
    o, lse = oracle.decode_gqa(w.q, w.k, w.v, 40, w.scale)
    o2, lse2 = oracle.decode_gqa(oracle.widen(w.q), oracle.widen(w.k[:, :, :40]),
                                 oracle.widen(w.v[:, :, :40]), 40, w.scale)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    assert np.all(np.isfinite(o))


# ------------------------------------------------------------------- backward ---
def _loss(q, k, v, dout, scale):
    """L = Σ O ∘ dO, whose gradient with respect to O is dO."""
    o, _ = oracle.prefill_causal(q, k, v, scale)
    return float(np.sum(o * dout))


def test_backward_matches_central_differences():
    """The gradients are the derivatives of L = Σ O∘dO: central differences
    of the forward oracle (fp64, step 1e-5) at sampled elements of Q, K, V."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, N, D = 1, 4, 2, 9, 6
    q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D)))
    dout = rng.standard_normal((B, Hq, N, D))
    scale = 0.7
    dq, dk, dv = oracle.prefill_causal_backward(q, k, v, dout, scale)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0, 0), (0, 1, 4, 2), (0, x.shape[1] - 1, N - 1, D - 1), (0, 0, N // 2, 3)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            lp = _loss(**{**args, name: xp}, dout=dout, scale=scale)
            lm = _loss(**{**args, name: xm}, dout=dout, scale=scale)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def test_backward_matches_torch_autograd():
    """Library special case: torch's CPU float64 SDPA (is_causal, contiguous
    GQA groups) differentiated by autograd."""
    import torch
    import torch.nn.functional as F
    w = workloads.gen_prefill(2, 6, 2, 37, 16, dtype="bf16", seed=23)
    rng = np.random.default_rng(4)
    dout = rng.standard_normal((2, 6, 37, 16))
    dq, dk, dv = oracle.prefill_causal_backward(w.q, w.k, w.v, dout, w.scale)
    q, k, v = (torch.from_numpy(oracle.widen(x)).requires_grad_() for x in (w.q, w.k, w.v))
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.scale, enable_gqa=True)
    o.backward(torch.from_numpy(dout))
    np.testing.assert_allclose(dq, q.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, k.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, v.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_closed_forms():
    """Equal value rows make O constant in Q and K: dQ = dK = 0. The last key
    is seen by the last query only: dV[N−1] = Σ_heads P[N−1,N−1]·dO[N−1].
    The first query sees key 0 alone (weight 1, no softmax gradient):
    dQ[0] = 0."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, N, D = 1, 4, 2, 11, 8
    q, k = rng.standard_normal((B, Hq, N, D)), rng.standard_normal((B, Hkv, N, D))
    v = np.repeat(rng.standard_normal((B, Hkv, 1, D)), N, axis=2)
    dout = rng.standard_normal((B, Hq, N, D))
    dq, dk, dv = oracle.prefill_causal_backward(q, k, v, dout, 0.5)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    v = rng.standard_normal((B, Hkv, N, D))
    dq, dk, dv = oracle.prefill_causal_backward(q, k, v, dout, 0.5)
    assert np.abs(dq[:, :, 0]).max() < 1e-14
    _, _, p = oracle.prefill_causal(q, k, v, 0.5, return_p=True)
    for hkv in range(Hkv):
        want = sum(p[0, h, N - 1, N - 1] * dout[0, h, N - 1] for h in (2 * hkv, 2 * hkv + 1))
        np.testing.assert_allclose(dv[0, hkv, N - 1], want, rtol=1e-14, atol=1e-15)


def test_backward_rows_equals_backward():
    """The row- and key-parallel backward (used for long sequences) gives the
    gradients of the serial one, which the three pins above fix: all rows and
    keys, and chosen subsets in any order, across GQA groups and ragged N."""
    for (B, Hq, Hkv, N, D, seed) in ((1, 4, 2, 9, 6, 1), (2, 6, 3, 40, 16, 2), (1, 2, 1, 1, 8, 3)):
        w = workloads.gen_prefill(B, Hq, Hkv, N, D, dtype="bf16", seed=seed)
        dout = workloads.gen_upstream_grad((B, Hq, N, D), seed=seed + 10)
        dq, dk, dv = oracle.prefill_causal_backward(w.q, w.k, w.v, dout, w.scale)
        rq, rk, rv = oracle.prefill_causal_backward_rows(w.q, w.k, w.v, dout, w.scale, threads=3)
        for a, b in ((rq, dq), (rk, dk), (rv, dv)):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
        rows, keys = [N - 1, 0, N // 2], [N // 3, N - 1]
        sq, sk, sv = oracle.prefill_causal_backward_rows(w.q, w.k, w.v, dout, w.scale, rows=rows,
                                                         keys=keys)
        np.testing.assert_array_equal(sq, rq[:, :, rows])
        np.testing.assert_array_equal(sk, rk[:, :, keys])
        np.testing.assert_array_equal(sv, rv[:, :, keys])


def test_bf16_widening_every_bit_pattern():
    """oracle.widen reads bfloat16 storage: every one of the 65,536 bit
    patterns widens to the value torch's bfloat16 → float64 conversion
    gives (the upper half of an IEEE binary32 word: sign, 8 exponent bits,
    7 mantissa bits), NaN patterns to NaN, ±0 and ±inf kept."""
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # spot values fixed by the format itself
    assert got[0x3F80] == 1.0 and got[0xBF80] == -1.0 and got[0x4049] == 3.140625
    assert got[0x0001] == 2.0 ** -133 and got[0x7F7F] == (2 - 2 ** -7) * 2.0 ** 127
    assert np.isinf(got[0x7F80]) and got[0xFF80] < 0 and np.isnan(got[0x7FC0])
