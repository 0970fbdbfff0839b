"""C-ABI checks that need no GPU: the library loads, exports every function
include/attn.h declares, and rejects invalid arguments on the host before
anything is enqueued (these calls return before any HIP call is made)."""
import ctypes
import os
import re

import pytest

import transformer_attention_05_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULLP, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4
P = 4096  # a fake, 16-byte aligned, non-null device address: never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return attn.load()


def test_header_symbols_exported(lib):
    names = _declared_functions()
    assert len(names) == 18, names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in [(0, "ATTN_OK"), (1, "ATTN_ERR_NULL_POINTER"), (2, "ATTN_ERR_BAD_SHAPE"),
                       (3, "ATTN_ERR_UNSUPPORTED"), (4, "ATTN_ERR_WORKSPACE"), (5, "ATTN_ERR_HIP")]:
        assert attn.status_string(code) == name


def _prefill(lib, dtype=0, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, N=64, D=64, scale=0.125):
    return lib.attn_prefill_causal(dtype, q, k, v, o, lse, B, Hq, Hkv, N, D, scale, None)


BAD_SCALES = (0.0, -0.125, float("inf"), float("nan"))


def test_prefill_validation(lib):
    assert _prefill(lib, q=None) == NULLP
    assert "NULL" in attn.last_error()
    assert _prefill(lib, lse=None) == NULLP
    assert _prefill(lib, N=0) == SHAPE
    assert _prefill(lib, B=0) == SHAPE
    assert _prefill(lib, Hq=3, Hkv=2) == SHAPE
    assert _prefill(lib, D=96) == UNSUP
    assert _prefill(lib, dtype=7) == UNSUP
    assert _prefill(lib, q=P + 2) == UNSUP              # misaligned
    assert _prefill(lib, B=1 << 12, Hq=64, Hkv=8, N=1 << 16, D=128) == SHAPE  # > 2^31 elements
    for s in BAD_SCALES:  # the kernels need a finite, positive scale
        assert _prefill(lib, scale=s) == SHAPE
        assert "scale" in attn.last_error()


def _gqa(lib, q=P, k=P, v=P, o=P, lse=P, B=2, Hq=8, Hkv=2, kv_len=100, kv_cap=128, D=128,
         ws=P, ws_bytes=1 << 30, scale=0.1):
    return lib.attn_decode_gqa(q, k, v, o, lse, B, Hq, Hkv, kv_len, kv_cap, D, scale, ws,
                               ws_bytes, None)


def test_decode_gqa_validation(lib):
    assert _gqa(lib, k=None) == NULLP
    assert _gqa(lib, kv_len=0) == SHAPE
    assert _gqa(lib, kv_len=129) == SHAPE
    assert _gqa(lib, Hq=6, Hkv=4) == SHAPE
    assert _gqa(lib, D=64) == UNSUP
    assert _gqa(lib, Hq=64, Hkv=2) == UNSUP             # group of 32 > 16
    for s in BAD_SCALES:
        assert _gqa(lib, scale=s) == SHAPE
    need = attn.attn_decode_gqa_workspace_bytes(2, 8, 2, 100, 128)
    assert need > 0
    assert _gqa(lib, ws=None) == WS
    assert _gqa(lib, ws_bytes=need - 1) == WS
    assert "workspace" in attn.last_error()


def test_backward_workspace_query():
    # D and LSE·log2(e) per query row, fp32, rows padded to the 32-row tile:
    # 2 arrays × (2·4 heads) × 128 rows × 4 B
    assert attn.attn_prefill_causal_backward_workspace_bytes(2, 4, 100, 128) == 8192


def test_decode_gqa_workspace_query():
    assert attn.attn_decode_gqa_workspace_bytes(8, 32, 8, 4096, 128) > 0
    assert attn.attn_decode_gqa_workspace_bytes(8, 32, 8, 4096, 64) == 0
    assert attn.attn_decode_gqa_workspace_bytes(8, 30, 8, 4096, 128) == 0
    assert attn.attn_decode_gqa_workspace_bytes(8, 32, 8, 0, 128) == 0


def test_decode_gqa_fp8_validation(lib):
    f = lambda **kw: lib.attn_decode_gqa_fp8(*[kw.get(n, d) for n, d in (
        ("q", P), ("k", P), ("v", P), ("o", P), ("lse", P), ("B", 2), ("Hq", 8), ("Hkv", 2),
        ("kv_len", 100), ("kv_cap", 128), ("D", 128), ("scale", 0.1), ("ws", P),
        ("ws_bytes", 1 << 30), ("st", None))])
    assert f(v=None) == NULLP
    assert f(kv_len=129) == SHAPE and f(kv_len=0) == SHAPE
    assert f(D=64) == UNSUP
    assert f(k=P + 8) == UNSUP
    assert f(ws_bytes=attn.attn_decode_gqa_workspace_bytes(2, 8, 2, 100) - 1) == WS
    for s in BAD_SCALES:
        assert f(scale=s) == SHAPE


def test_prefill_backward_validation(lib):
    f = lambda **kw: lib.attn_prefill_causal_backward(*[kw.get(n, d) for n, d in (
        ("q", P), ("k", P), ("v", P), ("o", P), ("lse", P), ("do", P), ("dq", P), ("dk", P),
        ("dv", P), ("B", 1), ("Hq", 8), ("Hkv", 2), ("N", 300), ("D", 128), ("scale", 0.1),
        ("ws", P), ("ws_bytes", 1 << 30), ("st", None))])
    assert f(do=None) == NULLP and f(dk=None) == NULLP
    assert f(N=0) == SHAPE and f(Hq=6, Hkv=4) == SHAPE
    assert f(D=64) == UNSUP and f(dv=P + 4) == UNSUP
    need = attn.attn_prefill_causal_backward_workspace_bytes(1, 8, 300, 128)
    assert need >= 4 * 8 * 300 and attn.attn_prefill_causal_backward_workspace_bytes(1, 8, 300, 64) == 0
    assert f(ws_bytes=need - 1) == WS
    for s in BAD_SCALES:
        assert f(scale=s) == SHAPE


def _mla(lib, q=P, c=P, o=P, lse=P, B=2, Hq=128, kv_len=1000, kv_cap=1024, Dqk=576, Dv=512,
         ws=P, ws_bytes=1 << 30, scale=0.07):
    return lib.attn_decode_mla_absorbed(q, c, o, lse, B, Hq, kv_len, kv_cap, Dqk, Dv, scale,
                                        ws, ws_bytes, None)


def test_decode_mla_validation(lib):
    assert _mla(lib, c=None) == NULLP
    assert _mla(lib, kv_len=1025) == SHAPE
    assert _mla(lib, kv_len=0) == SHAPE
    assert _mla(lib, Dqk=512, Dv=576) == SHAPE
    assert _mla(lib, Dqk=192, Dv=128) == UNSUP
    assert _mla(lib, Hq=20) == UNSUP
    for s in BAD_SCALES:
        assert _mla(lib, scale=s) == SHAPE
    need = attn.attn_decode_mla_workspace_bytes(2, 128, 1000)
    assert need > 0
    assert _mla(lib, ws_bytes=need - 1) == WS


def test_decode_mla_fp8_validation(lib):
    f = lambda **kw: lib.attn_decode_mla_fp8(*[kw.get(n, d) for n, d in (
        ("q", P), ("c", P), ("o", P), ("lse", P), ("B", 2), ("Hq", 128), ("kv_len", 1000),
        ("kv_cap", 1024), ("Dqk", 576), ("Dv", 512), ("scale", 0.07), ("ws", P),
        ("ws_bytes", 1 << 30), ("st", None))])
    assert f(c=None) == NULLP and f(lse=None) == NULLP
    assert f(kv_len=1025) == SHAPE and f(kv_len=0) == SHAPE
    assert f(Dqk=512, Dv=576) == SHAPE
    assert f(Dqk=192, Dv=128) == UNSUP and f(Hq=20) == UNSUP
    assert f(c=P + 8) == UNSUP                            # misaligned cache
    assert f(ws_bytes=attn.attn_decode_mla_workspace_bytes(2, 128, 1000) - 1) == WS
    for s in BAD_SCALES:
        assert f(scale=s) == SHAPE
    assert "attn_decode_mla_fp8" in attn.last_error()


def test_decode_mla_ragged_fp8_validation(lib):
    f = lambda **kw: lib.attn_decode_mla_ragged_fp8(*[kw.get(n, d) for n, d in (
        ("q", P), ("c", P), ("o", P), ("lse", P), ("lens", P), ("B", 2), ("Hq", 128),
        ("max_len", 1000), ("kv_cap", 1024), ("Dqk", 576), ("Dv", 512), ("scale", 0.07),
        ("ws", P), ("ws_bytes", 1 << 30), ("st", None))])
    assert f(lens=None) == NULLP and f(c=None) == NULLP
    assert f(max_len=1025) == SHAPE and f(max_len=0) == SHAPE
    assert f(Dqk=192, Dv=128) == UNSUP and f(Hq=20) == UNSUP
    assert f(c=P + 8) == UNSUP and f(lens=P + 2) == UNSUP   # misaligned cache, lengths
    assert f(ws_bytes=attn.attn_decode_mla_ragged_workspace_bytes(2, 128, 1000) - 1) == WS
    for s in BAD_SCALES:
        assert f(scale=s) == SHAPE
    assert "attn_decode_mla_ragged_fp8" in attn.last_error()


def _chunked(lib, q=P, k=P, v=P, o=P, lse=P, lens=P, B=2, Hq=8, Hkv=2, Nq=100, kv_cap=512,
             D=128, scale=0.1, ws=P, ws_bytes=1 << 30):
    return lib.attn_prefill_chunked(q, k, v, o, lse, lens, B, Hq, Hkv, Nq, kv_cap, D, scale, ws,
                                    ws_bytes, None)


def test_prefill_chunked_validation(lib):
    assert _chunked(lib, lens=None) == NULLP
    assert _chunked(lib, v=None) == NULLP
    assert _chunked(lib, Nq=0) == SHAPE
    assert _chunked(lib, Nq=513) == SHAPE                # the chunk does not fit the cache
    assert _chunked(lib, Hq=6, Hkv=4) == SHAPE
    assert _chunked(lib, B=1 << 10, Hkv=8, Hq=8, kv_cap=1 << 12, Nq=1 << 12) == SHAPE
    assert _chunked(lib, D=64) == UNSUP
    assert _chunked(lib, lens=P + 2) == UNSUP            # misaligned length array
    for s in BAD_SCALES:
        assert _chunked(lib, scale=s) == SHAPE
    # a short chunk over a long cache splits the keys and needs a workspace
    need = attn.attn_prefill_chunked_workspace_bytes(1, 8, 100, 32768)
    assert need > 1 << 20 and attn.attn_prefill_chunked_workspace_bytes(4, 32, 4096, 32768) == 256
    assert _chunked(lib, B=1, kv_cap=32768, ws_bytes=need - 1) == WS
    assert _chunked(lib, ws=None) == WS


def _gqa_r(lib, q=P, k=P, v=P, o=P, lse=P, lens=P, B=2, Hq=8, Hkv=2, max_len=100, kv_cap=128,
           D=128, ws=P, ws_bytes=1 << 30, scale=0.1):
    return lib.attn_decode_gqa_ragged(q, k, v, o, lse, lens, B, Hq, Hkv, max_len, kv_cap, D,
                                      scale, ws, ws_bytes, None)


def _mla_r(lib, q=P, c=P, o=P, lse=P, lens=P, B=2, Hq=128, max_len=1000, kv_cap=1024, Dqk=576,
           Dv=512, ws=P, ws_bytes=1 << 30, scale=0.07):
    return lib.attn_decode_mla_ragged(q, c, o, lse, lens, B, Hq, max_len, kv_cap, Dqk, Dv, scale,
                                      ws, ws_bytes, None)


def test_ragged_decode_validation(lib):
    assert _gqa_r(lib, lens=None) == NULLP
    assert _gqa_r(lib, max_len=0) == SHAPE
    assert _gqa_r(lib, max_len=129) == SHAPE
    assert "max_kv_len" in attn.last_error()
    assert _gqa_r(lib, D=64) == UNSUP
    assert _gqa_r(lib, lens=P + 1) == UNSUP
    need = attn.attn_decode_gqa_workspace_bytes(2, 8, 2, 100, 128)
    assert _gqa_r(lib, ws_bytes=need - 1) == WS
    assert _mla_r(lib, lens=None) == NULLP
    assert _mla_r(lib, max_len=1025) == SHAPE
    assert _mla_r(lib, Hq=20) == UNSUP
    need = attn.attn_decode_mla_ragged_workspace_bytes(2, 128, 1000)
    assert need > 0 and attn.attn_decode_mla_ragged_workspace_bytes(2, 120, 1000) == 0
    assert _mla_r(lib, ws_bytes=need - 1) == WS
    for s in BAD_SCALES:
        assert _gqa_r(lib, scale=s) == SHAPE and _mla_r(lib, scale=s) == SHAPE


def test_last_error_is_thread_local(lib):
    import threading
    assert _prefill(lib, q=None) == NULLP
    seen = []
    t = threading.Thread(target=lambda: seen.append(attn.last_error()))
    t.start()
    t.join()
    assert seen == [""]
    assert "NULL" in attn.last_error()


# ----------------------------------------------- Python binding checks (CPU) ---
def test_binding_requires_scale():
    """Every entry point takes the score scale from the caller; the binding
    infers none (no 1/√D, no MLA head width)."""
    import inspect
    for name in ("attn_prefill_causal", "attn_prefill_causal_backward", "attn_decode_gqa",
                 "attn_decode_gqa_fp8", "attn_decode_gqa_ragged", "attn_decode_mla_absorbed",
                 "attn_decode_mla_fp8", "attn_decode_mla_ragged", "attn_prefill_chunked"):
        prm = inspect.signature(getattr(attn, name)).parameters["scale"]
        assert prm.default is inspect.Parameter.empty, name
    with pytest.raises(TypeError):
        attn._scale(None)
    assert attn._scale(0.125) == 0.125


def test_binding_tensor_checks():
    """The checks every caller-supplied tensor passes before a library call:
    dtype, number of dimensions, exact shape (an out=, lse= or gradient of the
    wrong shape would be written past its end), contiguity, device. CPU
    tensors stand in for GPU ones here (the GPU requirement itself is
    checked too)."""
    import torch
    t = torch.empty(2, 3, 4, dtype=torch.bfloat16)
    cpu = torch.device("cpu")
    attn._check_tensor(t, "x", torch.bfloat16, shape=(2, 3, 4), device=cpu, cuda=False)
    with pytest.raises(TypeError, match="GPU"):
        attn._check_tensor(t, "x", torch.bfloat16)
    with pytest.raises(TypeError, match="float32"):
        attn._check_tensor(t, "x", torch.float32, cuda=False)
    with pytest.raises(ValueError, match="3-d"):
        attn._check_tensor(t, "x", torch.bfloat16, ndim=4, cuda=False)
    with pytest.raises(ValueError, match="shape"):
        attn._check_tensor(t, "out", torch.bfloat16, shape=(2, 3, 5), cuda=False)
    with pytest.raises(ValueError, match="contiguous"):
        attn._check_tensor(t.transpose(0, 1), "x", torch.bfloat16, cuda=False)
    with pytest.raises(ValueError, match="on"):
        attn._check_tensor(t, "x", torch.bfloat16, device=torch.device("meta"), cuda=False)
    with pytest.raises(TypeError):
        attn._check_tensor(t.numpy, "x", torch.bfloat16, cuda=False)
    # E4M3 tensors are passed on as their bytes
    f8 = torch.zeros(4, dtype=torch.float8_e4m3fn)
    assert attn._fp8_bytes(f8).dtype == torch.uint8
