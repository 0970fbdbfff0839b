"""Backward of the causal prefill on the GPU (through the C ABI) against the
fp64 oracle's gradients.

Comparison rule for gradients, derived by emulating the kernels' roundings
in fp64 (bf16 weights P into dV, bf16 dS into dK and dQ, D = rowsum(dO ∘ O)
from the forward's bf16 O, one bf16 rounding of each output) at N = 64, 129,
513 and on the 4k workload's first group. Each gradient row (a query row of
dQ, a key row of dK or dV) is a sum over its visible pairs, so part of its
error scales with the row's own size, which varies by an order of magnitude
along a long sequence (early queries see few keys); the error of D enters
every row of a head alike. Emulated: at most 0.018·(rms_row + rms_head)
beyond one bf16 ulp, and a mean of 2.3e-3 of the mean magnitude. Rule, per
tensor and (batch, head): |g − g_ref| ≤ ulp_bf16(|g_ref|) +
0.1·(rms_row(g_ref) + rms_head(g_ref)) + 1e-4 element-wise (rms_row over the
row's D entries, rms_head over the whole head), and
mean |g − g_ref| ≤ 5e-3 · mean |g_ref| + 1e-5; no NaN or Inf. The absolute
floors cover gradients that vanish identically, like dQ with one visible key,
where the kernel leaves fp32 rounding residue (≈ 1e-7)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import dev_bf16, host, ulp_bf16

pytestmark = pytest.mark.gpu


def check_grad(g, ref, what):
    g, ref = np.asarray(g, np.float64), np.asarray(ref, np.float64)
    assert g.shape == ref.shape and np.all(np.isfinite(g)), what
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            e, r = np.abs(g[b, h] - ref[b, h]), ref[b, h]
            rms = np.sqrt(np.mean(r ** 2, axis=-1, keepdims=True))
            tol = ulp_bf16(r) + 0.1 * (rms + np.sqrt(np.mean(r ** 2))) + 1e-4
            bad = e > tol
            if bad.any():
                i = np.unravel_index(np.argmax(e - tol), e.shape)
                raise AssertionError("%s (b=%d, h=%d): %d elements; worst at %s: err %g, |ref| %g, "
                                     "row rms %g" % (what, b, h, int(bad.sum()), i, e[i],
                                                     abs(r[i]), rms[i[0], 0]))
            assert e.mean() <= 5e-3 * np.abs(r).mean() + 1e-5, "%s (b=%d, h=%d): mean %g vs %g" % (
                what, b, h, e.mean(), np.abs(r).mean())


def _run(gpu, w, dout):
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    o, lse = gpu.attn_prefill_causal(q, k, v, w.scale)
    grads = gpu.attn_prefill_causal_backward(q, k, v, o, lse, dev_bf16(dout), w.scale)
    torch.cuda.synchronize()
    return grads


@pytest.mark.parametrize("B,Hq,Hkv,N", [
    (1, 1, 1, 1), (1, 2, 1, 5), (2, 4, 2, 64), (1, 8, 2, 100), (2, 4, 4, 129),
    (1, 4, 1, 300), (1, 8, 8, 257), (1, 2, 2, 513)])
def test_prefill_backward_matches_oracle(gpu, B, Hq, Hkv, N):
    """Ragged lengths (tiles of 32 queries and 128 keys with partial last
    ones), GQA groups 1..4, the single-token case."""
    w = workloads.gen_prefill(B, Hq, Hkv, N, 128, dtype="bf16", seed=N + Hq)
    dout = workloads.gen_upstream_grad((B, Hq, N, 128), seed=N + 7)
    dq, dk, dv = _run(gpu, w, dout)
    rq, rk, rv = oracle.prefill_causal_backward(w.q, w.k, w.v, dout, w.scale)
    check_grad(host(dq), rq, "dq %s" % ((B, Hq, Hkv, N),))
    check_grad(host(dk), rk, "dk %s" % ((B, Hq, Hkv, N),))
    check_grad(host(dv), rv, "dv %s" % ((B, Hq, Hkv, N),))


def test_prefill_backward_deterministic(gpu):
    w = workloads.gen_prefill(1, 8, 2, 333, 128, dtype="bf16", seed=5)
    dout = workloads.gen_upstream_grad((1, 8, 333, 128), seed=6)
    a, b = _run(gpu, w, dout), _run(gpu, w, dout)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_prefill_backward_4k_workload(gpu):
    """The 4k prefill workload in full (B=4, 32/8 heads, N=4096): finite
    gradients; two identities that hold at any size (every row of dS sums to
    0, so Σ_j dK_j = 0; every row of P sums to 1, so Σ_j dV_j = Σ over the
    group's heads of Σ_i dO_i); and every element of two (b, K/V head)
    groups against the oracle."""
    w = workloads.make("prefill_bf16_4k")
    dout = workloads.gen_upstream_grad((w.B, w.Hq, w.N, w.D), seed=1010)
    dq, dk, dv = _run(gpu, w, dout)
    for g in (dq, dk, dv):
        assert bool(torch.isfinite(g.float()).all())
    dk64, dv64 = host(dk), host(dv)
    G = w.Hq // w.Hkv
    do64 = oracle.widen(dout).reshape(w.B, w.Hkv, G, w.N, w.D)
    want_v = do64.sum(axis=(2, 3))
    got_v, got_k = dv64.sum(axis=2), dk64.sum(axis=2)
    scale_v = np.abs(dv64).sum(axis=2)
    assert np.all(np.abs(got_v - want_v) <= 1e-2 * scale_v + 1e-3)
    assert np.all(np.abs(got_k) <= 1e-2 * np.abs(dk64).sum(axis=2) + 1e-3)
    # element-wise parity on two (b, K/V head) groups of the full call: the
    # first and the last, every row of dQ and every key of dK, dV
    for b, hkv in ((0, 0), (w.B - 1, w.Hkv - 1)):
        hs = slice(G * hkv, G * (hkv + 1))
        rq, rk, rv = oracle.prefill_causal_backward_rows(
            w.q[b:b + 1, hs], w.k[b:b + 1, hkv:hkv + 1], w.v[b:b + 1, hkv:hkv + 1],
            dout[b:b + 1, hs], w.scale)
        what = "4k backward group (b=%d, hkv=%d)" % (b, hkv)
        check_grad(host(dq[b:b + 1, hs]), rq, "dq " + what)
        check_grad(dk64[b:b + 1, hkv:hkv + 1], rk, "dk " + what)
        check_grad(dv64[b:b + 1, hkv:hkv + 1], rv, "dv " + what)
