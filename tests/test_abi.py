"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects every invalid request on the host before any HIP call
(so these tests never touch a device; all pointers are fake)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import exact_attention_128_amd as A
    return A.load()


def test_header_symbols_exported(lib):
    names = _declared()
    assert "attn_fwd" in names and "attn_bwd" in names
    raw = ctypes.CDLL(os.path.join(ROOT, "exact_attention_128_amd", "libattn.so"))
    for n in names:
        assert hasattr(raw, n), "symbol %s declared in attn.h but not exported" % n


def test_binding_signatures_cover_header():
    from exact_attention_128_amd import _lib
    assert sorted(_lib.SIGNATURES) == _declared()


P = 0x10000  # fake, 256-byte aligned "device" address: never dereferenced


def _fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, S=16, D=128, scale=0.1, causal=0):
    return lib.attn_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, None)


def test_fwd_validation(lib):
    assert _fwd(lib, q=None) == 1
    assert _fwd(lib, lse=None) == 1
    assert _fwd(lib, B=0) == 2
    assert _fwd(lib, H=-1) == 2
    assert _fwd(lib, S=0) == 2
    assert _fwd(lib, B=1 << 20, H=1 << 10, S=1 << 10) == 2  # >= 2^40 elements
    assert _fwd(lib, D=96) == 3
    assert _fwd(lib, D=256) == 3
    assert _fwd(lib, v=P + 8) == 4
    assert _fwd(lib, lse=P + 2) == 4
    assert _fwd(lib, scale=float("inf")) == 6
    assert _fwd(lib, scale=float("nan")) == 6
    assert lib.attn_fwd_ex(P, P, P, P, P, 1, 1, 16, 128, 0.1, 0, -1.0, None) == 6
    assert lib.attn_fwd_ex(P, P, P, P, P, 1, 1, 16, 128, 0.1, 0, 65.0, None) == 6
    assert lib.attn_fwd_ex(P, P, P, P, P, 1, 1, 16, 128, 0.1, 0, float("nan"), None) == 6
    ev = lib.attn_fwd_rescale_events
    assert ev(P, P, P, P, P, 1, 1, 16, 128, 0.1, 0, 32.0, None, None) == 1
    assert ev(P, P, P, P, P, 1, 1, 16, 128, 0.1, 0, 32.0, P + 4, None) == 4
    assert ev(P, P, P, P, P, 1, 1, 16, 96, 0.1, 0, 32.0, P, None) == 3
    assert ev(P, P, P, P, P, 1, 1, 16, 128, 0.1, 0, 70.0, P, None) == 6


def test_bwd_validation(lib):
    ws = lib.attn_bwd_workspace_size(1, 1, 16, 128)
    assert ws == 512  # one 64-row block of (LSE*log2e, -Delta)
    assert lib.attn_bwd_workspace_size(0, 1, 16, 128) == 0
    assert lib.attn_bwd_workspace_size(1, 1, 16, 80) == 0

    def bwd(ws_ptr=P, ws_bytes=ws, D=128, S=16, **kw):
        ptrs = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P)
        ptrs.update(kw)
        return lib.attn_bwd(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["o"], ptrs["lse"], ptrs["do"],
                            ptrs["dq"], ptrs["dk"], ptrs["dv"], ws_ptr, ws_bytes, 1, 1, S, D,
                            0.1, 1, None)

    assert bwd(do=None) == 1
    assert bwd(ws_ptr=None) == 1
    assert bwd(S=0) == 2
    assert bwd(D=32) == 3
    assert bwd(dk=P + 4) == 4
    assert bwd(ws_ptr=P + 16) == 4
    assert bwd(ws_bytes=ws - 1) == 5


def test_strerror_covers_codes(lib):
    seen = set()
    for code in range(9):
        s = lib.attn_strerror(code)
        assert s and s.decode() not in seen
        seen.add(s.decode())
    assert lib.attn_strerror(1234) == b"unknown status code"
    assert lib.attn_version() >= 100


def test_python_binding_rejects_cpu_tensors():
    import torch
    import exact_attention_128_amd as A
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.fwd(q, q, q)
    with pytest.raises(TypeError):
        A.fwd(q.float(), q, q)
