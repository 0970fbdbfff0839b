"""fp64 CPU oracle for fused attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. The GPU library never calls it and shares no code with it.

The arithmetic lives in attn_oracle.c (plain loops, fp64, three-pass safe
softmax with an explicit causal mask; its header gives the definition and
the page citations). This wrapper only widens the stored inputs to float64
exactly, builds the C file with gcc when needed, and marshals arrays.

Inputs are numpy arrays: float32/float64 values, or uint16 arrays holding
bfloat16 bit patterns. Outputs are float64.

Parity pins live in tests/test_oracle_pins.py; every function here is pinned
there (page-printed values, closed forms, a library special case, brute
force on tiny inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_attn_oracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile attn_oracle.c into _attn_oracle.so (gcc, no FMA contraction)."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            dp = ctypes.POINTER(ctypes.c_double)
            ip = ctypes.POINTER(ctypes.c_int)
            i, d = ctypes.c_int, ctypes.c_double
            lib.oracle_prefill_causal.argtypes = [dp, dp, dp, i, i, i, i, i, d, ip, i,
                                                  dp, dp, dp, i]
            lib.oracle_decode_gqa.argtypes = [dp, dp, dp, i, i, i, i, i, i, d, dp, dp, dp, i]
            lib.oracle_decode_mla.argtypes = [dp, dp, i, i, i, i, i, i, d, dp, dp, i]
            lib.oracle_prefill_causal_backward.argtypes = [dp, dp, dp, dp, i, i, i, i, i, d,
                                                           dp, dp, dp, i]
            lib.oracle_prefill_causal_backward_rows.argtypes = [dp, dp, dp, dp, i, i, i, i, i, d,
                                                                ip, i, ip, i, dp, dp, dp, i]
            lib.oracle_prefill_chunked.argtypes = [dp, dp, dp, i, i, i, i, ip, i, i, d, ip, i,
                                                   dp, dp, i]
            lib.oracle_decode_gqa_ragged.argtypes = [dp, dp, dp, i, i, i, ip, i, i, d, dp, dp, i]
            lib.oracle_decode_mla_ragged.argtypes = [dp, dp, i, i, ip, i, i, i, d, dp, dp, i]
            for f in (lib.oracle_prefill_causal, lib.oracle_decode_gqa, lib.oracle_decode_mla,
                      lib.oracle_prefill_chunked, lib.oracle_decode_gqa_ragged,
                      lib.oracle_decode_mla_ragged, lib.oracle_prefill_causal_backward,
                      lib.oracle_prefill_causal_backward_rows):
                f.restype = ctypes.c_int
            _lib = lib
    return _lib


def default_threads() -> int:
    """Cores this process may use: its affinity mask, capped by
    OMP_NUM_THREADS when that is set (a shared host's per-job CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def widen(x: np.ndarray) -> np.ndarray:
    """Stored values → float64, exactly. uint16 means bfloat16 bit patterns,
    uint8 means OCP FP8 E4M3 codes (sign, 4-bit exponent with bias 7, 3-bit
    mantissa; exponent 0 is subnormal, m·2^-9; S.1111.111 is NaN)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        f32 = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return np.ascontiguousarray(f32, dtype=np.float64)
    if x.dtype == np.uint8:
        c = x.astype(np.int64)
        e, m = (c >> 3) & 15, c & 7
        mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, e - 10))
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return np.ascontiguousarray(np.where(c >> 7, -mag, mag), dtype=np.float64)
    if x.dtype in (np.float32, np.float64):
        return np.ascontiguousarray(x, dtype=np.float64)
    raise TypeError("oracle inputs must be float32/float64, bf16 bits (uint16) or E4M3 codes (uint8)")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def _lens(kv_lens, B) -> np.ndarray:
    lens = np.ascontiguousarray(np.asarray(kv_lens).reshape(-1), dtype=np.int32)
    if lens.shape[0] != B:
        raise ValueError("kv_lens must hold one length per sequence")
    return lens


def prefill_causal(q, k, v, scale, rows=None, return_p=False, threads=None):
    """Causal prefill with N queries against N keys.

    q [B,Hq,N,D], k/v [B,Hkv,N,D]. `rows` selects query rows to evaluate
    (default: all). Returns (o [B,Hq,R,D], lse [B,Hq,R]) and p [B,Hq,R,N]
    when return_p is set, R = len(rows).
    """
    q = np.asarray(q)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, D) and v.shape == (B, Hkv, N, D)
    rows = np.arange(N, dtype=np.int32) if rows is None else np.asarray(rows, dtype=np.int32)
    R = rows.shape[0]
    if R < 1 or rows.min() < 0 or rows.max() >= N:
        raise ValueError("query rows must lie in [0, N)")
    q64 = widen(q[:, :, rows, :])
    k64, v64 = widen(k), widen(v)
    o = np.empty((B, Hq, R, D))
    lse = np.empty((B, Hq, R))
    p = np.empty((B, Hq, R, N)) if return_p else None
    rc = _load().oracle_prefill_causal(
        _ptr(q64), _ptr(k64), _ptr(v64), B, Hq, Hkv, N, D, float(scale),
        rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), R, _ptr(o), _ptr(lse),
        _ptr(p) if p is not None else None, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_prefill_causal rejected its arguments")
    return (o, lse, p) if return_p else (o, lse)


def decode_gqa(q, k_cache, v_cache, kv_len, scale, return_p=False, threads=None):
    """Single-query decode. q [B,Hq,D]; caches [B,Hkv,kv_cap,D] (only the
    first kv_len slots are read). Returns (o [B,Hq,D], lse [B,Hq]) [+ p]."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    _, Hkv, kv_cap, _ = k_cache.shape
    q64 = widen(q)
    # only the filled prefix is widened (and read)
    k64 = widen(k_cache[:, :, :kv_len])
    v64 = widen(v_cache[:, :, :kv_len])
    o = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    p = np.empty((B, Hq, kv_len)) if return_p else None
    rc = _load().oracle_decode_gqa(
        _ptr(q64), _ptr(k64), _ptr(v64), B, Hq, Hkv, int(kv_len), int(kv_len), D,
        float(scale), _ptr(o), _ptr(lse), _ptr(p) if p is not None else None,
        threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_decode_gqa rejected its arguments")
    return (o, lse, p) if return_p else (o, lse)


def decode_mla_absorbed(q, ckv, kv_len, dv, scale, threads=None):
    """Absorbed-MLA decode. q [B,Hq,Dqk]; ckv [B,kv_cap,Dqk]; key = whole
    row, value = first dv channels. Returns (o [B,Hq,dv], lse [B,Hq])."""
    q = np.asarray(q)
    B, Hq, Dqk = q.shape
    q64 = widen(q)
    c64 = widen(ckv[:, :kv_len])
    o = np.empty((B, Hq, dv))
    lse = np.empty((B, Hq))
    rc = _load().oracle_decode_mla(
        _ptr(q64), _ptr(c64), B, Hq, int(kv_len), int(kv_len), Dqk, int(dv),
        float(scale), _ptr(o), _ptr(lse), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_decode_mla rejected its arguments")
    return o, lse


def prefill_chunked(q, k_cache, v_cache, kv_lens, scale, rows=None, threads=None):
    """A chunk of Nq new tokens against a cache (bottom-right causal mask).

    q [B,Hq,Nq,D]; caches [B,Hkv,kv_cap,D]; kv_lens [B] with Nq <= kv_lens[b]
    <= kv_cap: sequence b's keys are its first kv_lens[b] slots, the last Nq
    of them the chunk's own. `rows` selects chunk rows (default: all).
    Returns (o [B,Hq,R,D], lse [B,Hq,R]).
    """
    q = np.asarray(q)
    B, Hq, Nq, D = q.shape
    _, Hkv, kv_cap, _ = k_cache.shape
    lens = _lens(kv_lens, B)
    rows = np.arange(Nq, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    R = rows.shape[0]
    n = int(lens.max())   # slots past every sequence's length are never read
    q64 = widen(q[:, :, rows, :])
    k64, v64 = widen(k_cache[:, :, :n]), widen(v_cache[:, :, :n])
    o = np.empty((B, Hq, R, D))
    lse = np.empty((B, Hq, R))
    rc = _load().oracle_prefill_chunked(
        _ptr(q64), _ptr(k64), _ptr(v64), B, Hq, Hkv, Nq, _iptr(lens), n, D, float(scale),
        _iptr(rows), R, _ptr(o), _ptr(lse), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_prefill_chunked rejected its arguments")
    return o, lse


def decode_gqa_ragged(q, k_cache, v_cache, kv_lens, scale, threads=None):
    """Decode of a ragged batch: sequence b reads its first kv_lens[b] slots
    (0 allowed: O = 0, LSE = −∞). Returns (o [B,Hq,D], lse [B,Hq])."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    _, Hkv, kv_cap, _ = k_cache.shape
    lens = _lens(kv_lens, B)
    n = max(1, int(lens.max()))
    q64 = widen(q)
    k64, v64 = widen(k_cache[:, :, :n]), widen(v_cache[:, :, :n])
    o = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    rc = _load().oracle_decode_gqa_ragged(
        _ptr(q64), _ptr(k64), _ptr(v64), B, Hq, Hkv, _iptr(lens), n, D, float(scale),
        _ptr(o), _ptr(lse), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_decode_gqa_ragged rejected its arguments")
    return o, lse


def decode_mla_ragged(q, ckv, kv_lens, dv, scale, threads=None):
    """Absorbed-MLA decode of a ragged batch (sequence b reads its first
    kv_lens[b] rows). Returns (o [B,Hq,dv], lse [B,Hq])."""
    q = np.asarray(q)
    B, Hq, Dqk = q.shape
    lens = _lens(kv_lens, B)
    n = max(1, int(lens.max()))
    q64 = widen(q)
    c64 = widen(ckv[:, :n])
    o = np.empty((B, Hq, dv))
    lse = np.empty((B, Hq))
    rc = _load().oracle_decode_mla_ragged(
        _ptr(q64), _ptr(c64), B, Hq, _iptr(lens), n, Dqk, int(dv), float(scale),
        _ptr(o), _ptr(lse), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_decode_mla_ragged rejected its arguments")
    return o, lse


def prefill_causal_backward(q, k, v, dout, scale, threads=None):
    """Gradients of the causal prefill for the upstream gradient dout of O.

    q, dout [B,Hq,N,D]; k, v [B,Hkv,N,D]. Returns (dq, dk, dv) in float64,
    dk/dv summed over the query heads sharing each K/V head."""
    q = np.asarray(q)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, D) and v.shape == k.shape and dout.shape == q.shape
    q64, k64, v64, d64 = widen(q), widen(k), widen(v), widen(dout)
    dq = np.empty((B, Hq, N, D))
    dk = np.empty((B, Hkv, N, D))
    dv = np.empty((B, Hkv, N, D))
    rc = _load().oracle_prefill_causal_backward(
        _ptr(q64), _ptr(k64), _ptr(v64), _ptr(d64), B, Hq, Hkv, N, D, float(scale),
        _ptr(dq), _ptr(dk), _ptr(dv), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_prefill_causal_backward rejected its arguments")
    return dq, dk, dv


def prefill_causal_backward_rows(q, k, v, dout, scale, rows=None, keys=None, threads=None):
    """The gradients of prefill_causal_backward at chosen query rows (dq) and
    chosen keys (dk, dv), with the work spread over rows and keys so a long
    sequence is affordable. Default: every row and every key.

    Returns (dq [B,Hq,R,D], dk [B,Hkv,K,D], dv [B,Hkv,K,D]) in float64."""
    q = np.asarray(q)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, D) and v.shape == k.shape and dout.shape == q.shape
    rows = np.arange(N, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    keys = np.arange(N, dtype=np.int32) if keys is None else np.ascontiguousarray(keys, dtype=np.int32)
    q64, k64, v64, d64 = widen(q), widen(k), widen(v), widen(dout)
    dq = np.empty((B, Hq, rows.shape[0], D))
    dk = np.empty((B, Hkv, keys.shape[0], D))
    dv = np.empty((B, Hkv, keys.shape[0], D))
    rc = _load().oracle_prefill_causal_backward_rows(
        _ptr(q64), _ptr(k64), _ptr(v64), _ptr(d64), B, Hq, Hkv, N, D, float(scale),
        _iptr(rows), rows.shape[0], _iptr(keys), keys.shape[0], _ptr(dq), _ptr(dk), _ptr(dv),
        threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_prefill_causal_backward_rows rejected its arguments")
    return dq, dk, dv
