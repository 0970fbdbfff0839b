"""Long decode scan ("MLA 矩阵乘法吸收的数值稳定性治理", §五: before an
absorbed-MLA decode is trusted, run it for at least 4096 autoregressive
steps and scan the softmax extremes). Every cache length t = 1..4096 is
decoded on the GPU with one fixed query per head; the rope channels of the
cache grow with position so the scores drift upwards and the running maximum
keeps moving, and a few keys are outliers. Checked at every step: finite
outputs, LSE non-decreasing in t (adding a key can only raise the
log-sum-exp), O inside the range of the values seen so far; at steps spread
over the whole scan, the oracle.""" 
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_bf16, dev_bf16, host, ulp_bf16

pytestmark = pytest.mark.gpu

STEPS = 4096


def test_mla_decode_scan_4096_steps(gpu):
    Hq = 32
    w = workloads.gen_decode_mla(1, Hq, STEPS, kv_cap=STEPS + 16, seed=77)
    x = oracle.widen(w.ckv[:, :STEPS])
    # the rope channels (part of the key, not of the value) grow with the
    # position, so the scores drift upwards, and every 509th key is an
    # outlier; the values stay O(1)
    x[..., w.Dv:] *= np.linspace(1.0, 6.0, STEPS)[None, :, None]
    x[:, ::509, w.Dv:] *= 4.0
    w.ckv[:, :STEPS] = workloads.round_to_bf16_bits(x)
    q, c = dev_bf16(w.q), dev_bf16(w.ckv)
    ws = torch.empty(gpu.attn_decode_mla_workspace_bytes(1, Hq, STEPS), dtype=torch.uint8,
                     device="cuda")
    o_all = torch.empty((STEPS, Hq, w.Dv), dtype=torch.bfloat16, device="cuda")
    l_all = torch.empty((STEPS, Hq), dtype=torch.float32, device="cuda")
    for t in range(1, STEPS + 1):
        gpu.attn_decode_mla_absorbed(q, c, t, w.Dv, w.scale, out=o_all[t - 1:t], lse=l_all[t - 1:t],
                                     ws=ws)
    torch.cuda.synchronize()
    o, lse = host(o_all), host(l_all)                                    # [t, head, ...]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))

    # LSE never falls as keys are added (up to fp32 rounding of the sums)
    drop = lse[:-1] - lse[1:]
    assert drop.max() <= 2e-6 * max(1.0, np.abs(lse).max()), drop.max()
    # O is a convex combination of the values seen so far
    v = oracle.widen(w.ckv[0, :STEPS, :w.Dv])
    run_max, run_min = np.maximum.accumulate(v, 0), np.minimum.accumulate(v, 0)
    slack = 2.0 ** -7 * np.maximum(np.abs(run_max), np.abs(run_min))
    assert np.all(o <= run_max[:, None, :] + slack[:, None, :])
    assert np.all(o >= run_min[:, None, :] - slack[:, None, :])

    # the softmax extremes of the scan (largest weight of each step), from
    # the fp64 scores and the kernel's LSE
    s = (oracle.widen(w.q[0]) @ oracle.widen(w.ckv[0, :STEPS]).T) * w.scale   # [head, key]
    smax = np.maximum.accumulate(s, axis=1).T                                # [t, head]
    p_top = np.exp(smax - lse)
    # (LSE is checked to 1e-4 relative, floored at 1)
    assert np.all(p_top <= np.exp(1e-4 * np.maximum(1.0, np.abs(lse)))) and np.all(p_top > 0.0)
    print("scan: LSE %.3f .. %.3f, top weight %.3g .. %.3g"
          % (lse.min(), lse.max(), p_top.min(), p_top.max()))

    # the oracle at steps spread over the whole scan
    steps = sorted(set([1, 2, 3, 31, 32, 33, 511, 512, 513] + list(range(640, STEPS + 1, 640))
                       + [STEPS - 1, STEPS]))
    for t in steps:
        o_ref, lse_ref = oracle.decode_mla_absorbed(w.q, w.ckv, t, w.Dv, w.scale)
        # what rounding the exact result once to bf16 alone costs: with two
        # or three keys the outputs are O(1) mixtures of a few value rows and
        # that floor reaches the mean gate itself (1.016e-3 at t = 2 here)
        floor = np.abs(oracle.widen(workloads.round_to_bf16_bits(o_ref)) - o_ref).mean()
        if floor <= 0.9e-3:
            check_bf16(o[t - 1][None], o_ref, lse[t - 1][None], lse_ref, "scan step %d" % t)
        else:
            err = np.abs(o[t - 1][None] - o_ref)
            assert np.all(err <= np.maximum(1e-2, ulp_bf16(o_ref))), "scan step %d" % t
            assert err.mean() <= 1.05 * floor, "scan step %d: mean %g, floor %g" % (t, err.mean(), floor)
            lrel = np.abs(lse[t - 1][None] - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
            assert lrel.max() <= 1e-4, "scan step %d" % t
