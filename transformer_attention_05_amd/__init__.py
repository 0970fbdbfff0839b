"""MI355X (gfx950) fused attention: thin Python binding over libattn.so.

The functions carry the names of the C ABI (include/attn.h) and do argument
marshalling only: every step of attention runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream, nothing else. There is
no fallback: if libattn.so is missing or fails to load, every call raises.

    o, lse = attn_prefill_causal(q, k, v, scale)                  # [B,H,N,D]
    o, lse = attn_decode_gqa(q, k_cache, v_cache, kv_len, scale)  # q [B,Hq,D]
    o, lse = attn_decode_mla_absorbed(q, ckv, kv_len, 512, scale) # q [B,Hq,576]
    o, lse = attn_prefill_chunked(q, k_cache, v_cache, kv_lens, scale)  # q [B,Hq,Nq,D]
    o, lse = attn_decode_gqa_ragged(q, k_cache, v_cache, kv_lens, max_kv_len, scale)
    o, lse = attn_decode_mla_ragged(q, ckv, kv_lens, max_kv_len, 512, scale)
    o, lse = attn_decode_gqa_fp8(q, k_fp8, v_fp8, kv_len, scale)   # E4M3 caches (uint8)
    o, lse = attn_decode_mla_fp8(q, ckv_fp8, kv_len)                 # E4M3 latent cache
    dq, dk, dv = attn_prefill_causal_backward(q, k, v, o, lse, dout, scale)
(kv_lens: an int32 GPU tensor of per-sequence lengths, read by the kernels.)
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_OK, ATTN_BF16, ATTN_FP32 = 0, 0, 1

_lib = None
_lock = threading.Lock()
_workspaces: dict = {}


class AttnError(RuntimeError):
    """A non-OK status from libattn.so (carries the status code)."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load() -> ctypes.CDLL:
    """Load the in-tree libattn.so (built by build.py); raise if absent."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libattn.so not found at %s: build it with "
                "`python -m transformer_attention_05_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.attn_prefill_causal.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.attn_decode_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
        lib.attn_decode_mla_absorbed.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
        lib.attn_decode_gqa_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
        lib.attn_decode_mla_fp8.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
        lib.attn_prefill_causal_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i,
                                                     i, f, vp, sz, vp]
        lib.attn_prefill_causal_backward_workspace_bytes.argtypes = [i, i, i, i]
        lib.attn_prefill_causal_backward_workspace_bytes.restype = sz
        lib.attn_prefill_chunked.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
        lib.attn_prefill_chunked_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.attn_prefill_chunked_workspace_bytes.restype = sz
        lib.attn_decode_gqa_ragged.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz,
                                               vp]
        lib.attn_decode_mla_ragged.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
        lib.attn_decode_gqa_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.attn_decode_mla_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.attn_decode_mla_ragged_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.attn_decode_gqa_workspace_bytes.restype = sz
        lib.attn_decode_mla_workspace_bytes.restype = sz
        lib.attn_decode_mla_ragged_workspace_bytes.restype = sz
        for fn in (lib.attn_prefill_causal, lib.attn_decode_gqa, lib.attn_decode_mla_absorbed,
                   lib.attn_prefill_chunked, lib.attn_decode_gqa_ragged, lib.attn_decode_gqa_fp8,
                   lib.attn_prefill_causal_backward,
                   lib.attn_decode_mla_ragged, lib.attn_decode_mla_fp8):
            fn.restype = ctypes.c_int
        lib.attn_status_string.argtypes = [i]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(status: int, lib) -> None:
    if status != ATTN_OK:
        name = lib.attn_status_string(status).decode()
        raise AttnError(status, "%s: %s" % (name, lib.attn_last_error().decode()))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %d-d tensor" % (name, ndim))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of at least nbytes for (device, current stream).

    It carries split partials between the two kernels of one decode call, so
    calls on one stream may share it and calls on different streams get
    different buffers. Allocate it outside any graph capture (a first call
    on the stream does that).
    """
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def attn_prefill_causal(q, k, v, scale=None, out=None, lse=None):
    """Causal prefill. q [B,Hq,N,D], k/v [B,Hkv,N,D] (bf16 or fp32, same
    dtype). Returns (o [B,Hq,N,D] same dtype, lse [B,Hq,N] fp32)."""
    lib = load()
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, dtype, 4)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, N, D] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "out", dtype, 4)
    _need(l, "lse", torch.float32, 3)
    st = lib.attn_prefill_causal(ATTN_BF16 if dtype == torch.bfloat16 else ATTN_FP32,
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l),
                                 B, Hq, Hkv, N, D, float(scale), _stream(q.device))
    _check(st, lib)
    return o, l


def attn_prefill_causal_backward(q, k, v, o, lse, dout, scale=None, dq=None, dk=None, dv=None,
                                 ws=None):
    """Backward of attn_prefill_causal (bf16, D = 128). q, o, dout [B,Hq,N,D];
    k, v [B,Hkv,N,D]; lse [B,Hq,N] fp32 from the forward. Returns (dq, dk, dv)."""
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, name, torch.bfloat16, 4)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shapes must be q/o/dout [B,Hq,N,D], k/v [B,Hkv,N,D]")
    _need(lse, "lse", torch.float32, 3)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, name, torch.bfloat16, 4)
    need = lib.attn_prefill_causal_backward_workspace_bytes(B, Hq, N, D)
    w = workspace(need, q.device) if ws is None else ws
    st = lib.attn_prefill_causal_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                          _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, N, D,
                                          float(scale), _ptr(w), w.numel() * w.element_size(),
                                          _stream(q.device))
    _check(st, lib)
    return dq, dk, dv


def attn_decode_gqa_workspace_bytes(B, Hq, Hkv, kv_len, D=128) -> int:
    return int(load().attn_decode_gqa_workspace_bytes(B, Hq, Hkv, kv_len, D))


def attn_prefill_causal_backward_workspace_bytes(B, Hq, N, D=128) -> int:
    return int(load().attn_prefill_causal_backward_workspace_bytes(B, Hq, N, D))


def attn_decode_gqa(q, k_cache, v_cache, kv_len, scale=None, out=None, lse=None, ws=None):
    """Single-query GQA decode. q [B,Hq,D] bf16; caches [B,Hkv,kv_cap,D] bf16
    filled to kv_len. Returns (o [B,Hq,D] bf16, lse [B,Hq] fp32)."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, D = q.shape
    _, Hkv, kv_cap, _ = k_cache.shape
    if k_cache.shape != (B, Hkv, kv_cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, kv_cap, D] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "out", torch.bfloat16, 3)
    _need(l, "lse", torch.float32, 2)
    need = lib.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, int(kv_len), D)
    w = workspace(need, q.device) if ws is None else ws
    st = lib.attn_decode_gqa(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(l),
                             B, Hq, Hkv, int(kv_len), kv_cap, D, float(scale),
                             _ptr(w), w.numel() * w.element_size(), _stream(q.device))
    _check(st, lib)
    return o, l


def attn_decode_gqa_fp8(q, k_cache, v_cache, kv_len, scale=None, out=None, lse=None, ws=None):
    """GQA decode over an FP8 E4M3 cache. q [B,Hq,D] bf16; caches
    [B,Hkv,kv_cap,D] torch.uint8 (E4M3 codes) or torch.float8_e4m3fn, filled
    to kv_len. Returns (o [B,Hq,D] bf16, lse [B,Hq] fp32)."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype == torch.float8_e4m3fn:
            t = t.view(torch.uint8)
        _need(t, name, torch.uint8, 4)
    B, Hq, D = q.shape
    _, Hkv, kv_cap, _ = k_cache.shape
    if k_cache.shape != (B, Hkv, kv_cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, kv_cap, D] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "out", torch.bfloat16, 3)
    _need(l, "lse", torch.float32, 2)
    need = lib.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, int(kv_len), D)
    w = workspace(need, q.device) if ws is None else ws
    st = lib.attn_decode_gqa_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(l),
                                 B, Hq, Hkv, int(kv_len), kv_cap, D, float(scale),
                                 _ptr(w), w.numel() * w.element_size(), _stream(q.device))
    _check(st, lib)
    return o, l


def attn_decode_mla_workspace_bytes(B, Hq, kv_len, Dqk=576, Dv=512) -> int:
    return int(load().attn_decode_mla_workspace_bytes(B, Hq, kv_len, Dqk, Dv))


def attn_decode_mla_ragged_workspace_bytes(B, Hq, max_kv_len, Dqk=576, Dv=512) -> int:
    return int(load().attn_decode_mla_ragged_workspace_bytes(B, Hq, max_kv_len, Dqk, Dv))


def attn_decode_mla_absorbed(q, ckv, kv_len, dv=512, scale=None, out=None, lse=None, ws=None):
    """Absorbed MLA decode. q [B,Hq,Dqk] bf16 (absorbed, channel-balanced
    query | rope), ckv [B,kv_cap,Dqk] bf16 (balanced latent | rope). Value =
    first dv channels of each cached row. Returns (o [B,Hq,dv] bf16, lse)."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(ckv, "ckv", torch.bfloat16, 3)
    B, Hq, Dqk = q.shape
    kv_cap = ckv.shape[1]
    if ckv.shape != (B, kv_cap, Dqk):
        raise ValueError("ckv must be [B, kv_cap, Dqk] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(128 + 64)
    o = torch.empty((B, Hq, dv), dtype=torch.bfloat16, device=q.device) if out is None else out
    l = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "out", torch.bfloat16, 3)
    _need(l, "lse", torch.float32, 2)
    need = lib.attn_decode_mla_workspace_bytes(B, Hq, int(kv_len), Dqk, dv)
    w = workspace(need, q.device) if ws is None else ws
    st = lib.attn_decode_mla_absorbed(_ptr(q), _ptr(ckv), _ptr(o), _ptr(l), B, Hq, int(kv_len),
                                      kv_cap, Dqk, dv, float(scale), _ptr(w),
                                      w.numel() * w.element_size(), _stream(q.device))
    _check(st, lib)
    return o, l


def attn_decode_mla_fp8(q, ckv, kv_len, dv=512, scale=None, out=None, lse=None, ws=None):
    """Absorbed MLA decode over an FP8 E4M3 latent cache. q [B,Hq,Dqk] bf16
    (absorbed, channel-balanced query | rope); ckv [B,kv_cap,Dqk]
    torch.uint8 (E4M3 codes of the balanced latent | rope) or
    torch.float8_e4m3fn. Returns (o [B,Hq,dv] bf16, lse [B,Hq] fp32)."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(ckv.view(torch.uint8) if ckv.dtype == torch.float8_e4m3fn else ckv, "ckv", torch.uint8, 3)
    B, Hq, Dqk = q.shape
    kv_cap = ckv.shape[1]
    if ckv.shape != (B, kv_cap, Dqk):
        raise ValueError("ckv must be [B, kv_cap, Dqk] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(128 + 64)
    o = torch.empty((B, Hq, dv), dtype=torch.bfloat16, device=q.device) if out is None else out
    l = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "out", torch.bfloat16, 3)
    _need(l, "lse", torch.float32, 2)
    need = lib.attn_decode_mla_workspace_bytes(B, Hq, int(kv_len), Dqk, dv)
    w = workspace(need, q.device) if ws is None else ws
    st = lib.attn_decode_mla_fp8(_ptr(q), _ptr(ckv), _ptr(o), _ptr(l), B, Hq, int(kv_len), kv_cap,
                                 Dqk, dv, float(scale), _ptr(w), w.numel() * w.element_size(),
                                 _stream(q.device))
    _check(st, lib)
    return o, l


def _need_lens(kv_lens, B):
    _need(kv_lens, "kv_lens", torch.int32, 1)
    if kv_lens.shape[0] != B:
        raise ValueError("kv_lens must hold one length per sequence")


def attn_prefill_chunked_workspace_bytes(B, Hq, Nq, kv_cap, D=128) -> int:
    return int(load().attn_prefill_chunked_workspace_bytes(B, Hq, Nq, kv_cap, D))


def attn_prefill_chunked(q, k_cache, v_cache, kv_lens, scale=None, out=None, lse=None, ws=None):
    """Chunked prefill against a cache. q [B,Hq,Nq,D] bf16; caches
    [B,Hkv,kv_cap,D] bf16 filled to kv_lens[b] (int32 GPU tensor [B], each
    in [Nq, kv_cap]), the last Nq slots being the chunk's own tokens.
    Returns (o [B,Hq,Nq,D] bf16, lse [B,Hq,Nq] fp32)."""
    lib = load()
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, Nq, D = q.shape
    _, Hkv, kv_cap, _ = k_cache.shape
    if k_cache.shape != (B, Hkv, kv_cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, kv_cap, D] matching q")
    _need_lens(kv_lens, B)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "out", torch.bfloat16, 4)
    _need(l, "lse", torch.float32, 3)
    need = lib.attn_prefill_chunked_workspace_bytes(B, Hq, Nq, kv_cap, D)
    w = workspace(need, q.device) if ws is None else ws
    st = lib.attn_prefill_chunked(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(l),
                                  _ptr(kv_lens), B, Hq, Hkv, Nq, kv_cap, D, float(scale),
                                  _ptr(w), w.numel() * w.element_size(), _stream(q.device))
    _check(st, lib)
    return o, l


def attn_decode_gqa_ragged(q, k_cache, v_cache, kv_lens, max_kv_len, scale=None, out=None,
                           lse=None, ws=None):
    """GQA decode of a ragged batch: sequence b's caches are filled to
    kv_lens[b] (int32 GPU tensor [B], each at most max_kv_len). Returns
    (o [B,Hq,D] bf16, lse [B,Hq] fp32); a sequence of length 0 gets O = 0,
    LSE = -inf."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, D = q.shape
    _, Hkv, kv_cap, _ = k_cache.shape
    if k_cache.shape != (B, Hkv, kv_cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, kv_cap, D] matching q")
    _need_lens(kv_lens, B)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "out", torch.bfloat16, 3)
    _need(l, "lse", torch.float32, 2)
    need = lib.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, int(max_kv_len), D)
    w = workspace(need, q.device) if ws is None else ws
    st = lib.attn_decode_gqa_ragged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(l),
                                    _ptr(kv_lens), B, Hq, Hkv, int(max_kv_len), kv_cap, D,
                                    float(scale), _ptr(w), w.numel() * w.element_size(),
                                    _stream(q.device))
    _check(st, lib)
    return o, l


def attn_decode_mla_ragged(q, ckv, kv_lens, max_kv_len, dv=512, scale=None, out=None, lse=None,
                           ws=None):
    """Absorbed MLA decode of a ragged batch: sequence b's latent cache is
    filled to kv_lens[b] (int32 GPU tensor [B], each at most max_kv_len).
    Returns (o [B,Hq,dv] bf16, lse [B,Hq] fp32)."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(ckv, "ckv", torch.bfloat16, 3)
    B, Hq, Dqk = q.shape
    kv_cap = ckv.shape[1]
    if ckv.shape != (B, kv_cap, Dqk):
        raise ValueError("ckv must be [B, kv_cap, Dqk] matching q")
    _need_lens(kv_lens, B)
    if scale is None:
        scale = 1.0 / math.sqrt(128 + 64)
    o = torch.empty((B, Hq, dv), dtype=torch.bfloat16, device=q.device) if out is None else out
    l = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "out", torch.bfloat16, 3)
    _need(l, "lse", torch.float32, 2)
    need = lib.attn_decode_mla_ragged_workspace_bytes(B, Hq, int(max_kv_len), Dqk, dv)
    w = workspace(need, q.device) if ws is None else ws
    st = lib.attn_decode_mla_ragged(_ptr(q), _ptr(ckv), _ptr(o), _ptr(l), _ptr(kv_lens), B, Hq,
                                    int(max_kv_len), kv_cap, Dqk, dv, float(scale), _ptr(w),
                                    w.numel() * w.element_size(), _stream(q.device))
    _check(st, lib)
    return o, l


def status_string(status: int) -> str:
    return load().attn_status_string(status).decode()


def last_error() -> str:
    return load().attn_last_error().decode()
