"""LDS race check on the GPU: the debug build libattn_lds_poison.so writes a NaN
pattern over every direct-to-LDS load's destination before issuing the load
(gfx950.h, lds_dma16).  Without a race its results are bit-identical to the
product library's on the same inputs; a piece read before its load's wait and
barrier, a refill that overtakes the piece's last reader, or a load that
leaves bytes unwritten (rows past the sequence end must land as zeros) shows
up as NaN or as a difference.  Every ring kernel is covered: the long and
short forwards, the FP8 forward, and both backward kernels."""
import os

import numpy as np
import pytest

import attn_inputs as ai
import parity as P

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POISON = os.path.join(ROOT, "exact_attention_128_amd", "libattn_lds_poison.so")


@pytest.fixture(scope="module")
def libs():
    from exact_attention_128_amd import _lib
    if not os.path.exists(POISON):
        pytest.fail("libattn_lds_poison.so is not built (exact_attention_128_amd/build.py)")
    return _lib.load(), _lib.open_library(POISON)


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _fwd(lib, q, k, v, causal, scale):
    import torch
    B, H, S, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    rc = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, H, S, D, scale, int(causal), _stream())
    assert rc == 0, rc
    torch.cuda.synchronize()
    return o, lse


def _bwd(lib, q, k, v, o, lse, do, causal, scale):
    import torch
    B, H, S, D = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    n = lib.attn_bwd_workspace_size(B, H, S, D)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    rc = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                      n, B, H, S, D, scale, int(causal), _stream())
    assert rc == 0, rc
    torch.cuda.synchronize()
    return dq, dk, dv


def _same_bits(a, b, what):
    import torch
    assert torch.isfinite(a.float()).all(), "%s: non-finite values" % what
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
        "%s: race-check build differs from the product library" % what


# (B, H, S, D): several query blocks and key steps with ragged tails, the
# first partial steps of the long kernel, and each packing of the short one
FWD_SHAPES = [(1, 3, 1000, 128), (2, 4, 1500, 64), (1, 2, 130, 128), (1, 2, 257, 64),
              (2, 3, 100, 128), (1, 7, 50, 64), (1, 9, 24, 128), (2, 5, 4100, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", FWD_SHAPES)
def test_forward_matches_product_bitwise(libs, shape, causal):
    import torch
    prod, poison = libs
    B, H, S, D = shape
    bits = ai.make_inputs(B, H, S, D, 3000 + S + D + int(causal))
    dev = torch.device("cuda", 0)
    q, k, v = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v"))
    scale = 1.0 / np.sqrt(D)
    o1, l1 = _fwd(prod, q, k, v, causal, scale)
    o2, l2 = _fwd(poison, q, k, v, causal, scale)
    print("fwd", shape, causal)
    _same_bits(o1, o2, "O %s causal=%s" % (shape, causal))
    _same_bits(l1, l2, "LSE %s causal=%s" % (shape, causal))


def test_forward_race_check_build_against_oracle(libs):
    """The race-check build on its own, every element against the oracle."""
    import torch
    _, poison = libs
    B, H, S, D = 1, 3, 777, 128
    bits = ai.make_inputs(B, H, S, D, 3100)
    dev = torch.device("cuda", 0)
    q, k, v = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v"))
    scale = 1.0 / np.sqrt(D)
    o, lse = _fwd(poison, q, k, v, True, scale)
    o64 = ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(o))
    o_ref, lse_ref = P.oracle_fwd_full(bits, True, scale)
    P.assert_fwd_ok(P.fwd_errors(o64, lse.cpu().numpy().astype(np.float64), o_ref, lse_ref),
                    "race-check build")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1100, 128), (2, 3, 333, 64), (1, 2, 4100, 128)])
def test_backward_matches_product_bitwise(libs, shape, causal):
    import torch
    prod, poison = libs
    B, H, S, D = shape
    bits = ai.make_inputs(B, H, S, D, 3200 + S + D + int(causal), with_dout=True)
    dev = torch.device("cuda", 0)
    q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
    scale = 1.0 / np.sqrt(D)
    o, lse = _fwd(prod, q, k, v, causal, scale)
    g1 = _bwd(prod, q, k, v, o, lse, do, causal, scale)
    g2 = _bwd(poison, q, k, v, o, lse, do, causal, scale)
    print("bwd", shape, causal)
    for name, a, b in zip(("dQ", "dK", "dV"), g1, g2):
        _same_bits(a, b, "%s %s causal=%s" % (name, shape, causal))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 3, 1000, 128), (1, 2, 2100, 64)])
def test_fp8_forward_matches_product_bitwise(libs, shape, causal):
    import torch
    prod, poison = libs
    B, H, S, D = shape
    b8 = ai.make_inputs_fp8(B, H, S, D, 3300 + S + D + int(causal))
    dev = torch.device("cuda", 0)
    q, k, v = (ai.to_torch_u8(b8[n], dev) for n in ("q", "k", "v"))
    scale = 1.0 / np.sqrt(D)
    outs = []
    for lib in (prod, poison):
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
        rc = lib.attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, S, D, scale, int(causal), b8["q_descale"],
                              b8["k_descale"], b8["v_descale"], _stream())
        assert rc == 0, rc
        torch.cuda.synchronize()
        outs.append((o, lse))
    print("fp8", shape, causal)
    _same_bits(outs[0][0], outs[1][0], "FP8 O %s causal=%s" % (shape, causal))
    _same_bits(outs[0][1], outs[1][1], "FP8 LSE %s causal=%s" % (shape, causal))
