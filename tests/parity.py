"""Helpers for GPU-vs-oracle parity tests: device upload of the seeded host
arrays and the comparison rule.

Comparison rule (bf16 outputs against the fp64 oracle):
  * element-wise |O − O_ref| ≤ max(1e-2, ulp_bf16(|O_ref|)), where
    ulp_bf16(x) = 2^(⌊log2 x⌋ − 7): the final rounding to bf16 alone can err
    by half that much, so for |O| ≥ 4 the flat 1e-2 is below the bf16 grid;
  * mean |O − O_ref| ≤ 1e-3;
  * LSE: |ΔLSE| / max(1, |LSE_ref|) ≤ 1e-4 (the floor avoids dividing by an
    LSE that happens to sit near 0);
  * no NaN or Inf anywhere.
fp32 outputs use max-abs ≤ 1e-4 and mean-abs ≤ 1e-5 with the same LSE rule.
"""
import numpy as np
import torch


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def dev_f32(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_bf16(o, o_ref, lse, lse_ref, what=""):
    """Assert the comparison rule; return a dict of the statistics."""
    o, o_ref, lse, lse_ref = (np.asarray(a, dtype=np.float64) for a in (o, o_ref, lse, lse_ref))
    assert o.shape == o_ref.shape and lse.shape == lse_ref.shape, what
    assert np.all(np.isfinite(o)), "%s: non-finite O" % what
    assert np.all(np.isfinite(lse)), "%s: non-finite LSE" % what
    err = np.abs(o - o_ref)
    tol = np.maximum(1e-2, ulp_bf16(o_ref))
    bad = err > tol
    lrel = np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                 n_ulp_only=int(np.sum((err > 1e-2) & ~bad)), lse_rel=float(lrel.max()))
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError("%s: %d elements beyond tolerance; worst at %s: got %r want %r"
                             % (what, int(bad.sum()), i, o[i], o_ref[i]))
    assert stats["mean_abs"] <= 1e-3, "%s: mean abs error %g" % (what, stats["mean_abs"])
    assert stats["lse_rel"] <= 1e-4, "%s: LSE rel error %g" % (what, stats["lse_rel"])
    return stats


def check_f32(o, o_ref, lse, lse_ref, what=""):
    o, o_ref, lse, lse_ref = (np.asarray(a, dtype=np.float64) for a in (o, o_ref, lse, lse_ref))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    err = np.abs(o - o_ref)
    lrel = np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
    assert err.max() <= 1e-4, "%s: max abs error %g" % (what, err.max())
    assert err.mean() <= 1e-5, "%s: mean abs error %g" % (what, err.mean())
    assert lrel.max() <= 1e-4, "%s: LSE rel error %g" % (what, lrel.max())
    return dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_rel=float(lrel.max()))


def check_bf16_channels(o, o_ref, lse, lse_ref, values, what=""):
    """The comparison rule applied channel by channel in units of that
    channel's values: O and O_ref are divided by g_c = 2^⌊log2 max_j |v_jc|⌋
    (a power of two, exact in float64), then check_bf16 applies. Each output
    channel is a convex combination of the values of that channel, so its
    error scales with their magnitude; this keeps the gate meaningful when
    channels span many decades (an un-balanced latent cache). `values`: the
    stored value rows, any leading shape, channels last."""
    v = np.abs(np.asarray(values, dtype=np.float64))
    vmax = v.reshape(-1, v.shape[-1]).max(axis=0)
    g = 2.0 ** np.floor(np.log2(np.maximum(vmax, 2.0 ** -126)))
    return check_bf16(np.asarray(o, np.float64) / g, np.asarray(o_ref, np.float64) / g,
                      lse, lse_ref, what)
