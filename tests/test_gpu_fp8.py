"""GPU parity of the FP8 (E4M3) forward against the fp64 oracle on the
dequantized inputs, to the bound its accuracy contract derives (parity.py:
E4M3 rounding of the weights, O normalised by the rounded sum, bf16 output,
fp32 accumulation) and LSE within 1e-3."""
import numpy as np
import pytest

import attn_inputs as ai
import parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 17, 130, 257, 1000])
def test_ragged_lengths(S, D, causal):
    bits = ai.make_inputs_fp8(1, 3, S, D, 3000 + S + D + int(causal))
    P.check_fp8(bits, causal, 1.0 / np.sqrt(D), what="fp8 S=%d D=%d causal=%s" % (S, D, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_multi_block_and_xcd_order(causal):
    """Several 256-row blocks and 128-key steps with a ragged tail; B*H = 8
    takes the XCD-aware block order."""
    bits = ai.make_inputs_fp8(2, 4, 1500, 128, 3100 + int(causal))
    P.check_fp8(bits, causal, 1.0 / np.sqrt(128), what="fp8 S=1500 causal=%s" % causal)


def test_rising_maximum():
    """Rising row maxima: the FP8 kernel rescales whenever a lane's step sum
    passes 2^8 (weights stay inside E4M3's range), many times per row here."""
    bits = ai.make_inputs_fp8(1, 3, 2100, 128, 3200, stress=True)
    P.check_fp8(bits, True, 1.0 / np.sqrt(128), what="fp8 rising maximum")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_scale_values(scale):
    bits = ai.make_inputs_fp8(1, 2, 300, 128, 3300)
    for causal in (False, True):
        P.check_fp8(bits, causal, scale, what="fp8 scale=%g causal=%s" % (scale, causal))


def test_large_score_jump():
    """One key ~150 nats above every earlier score: the weights against the
    stale maximum overflow to inf, the rescale recovers."""
    B, H, S, D = 1, 2, 700, 128
    rng = np.random.default_rng(3400)
    u = np.where(rng.random(D) < 0.5, -1.0, 1.0)
    q = np.broadcast_to(2.0 * u, (B, H, S, D)).astype(np.float32)
    k = rng.standard_normal((B, H, S, D)).astype(np.float32)
    k[:, :, 600, :] = 7.0 * u
    v = rng.standard_normal((B, H, S, D)).astype(np.float32)
    bits = {}
    for name, t in (("q", q), ("k", k), ("v", v)):
        bits[name], bits[name + "_descale"] = ai.quantize_e4m3(t)
    P.check_fp8(bits, True, 1.0 / np.sqrt(D), what="fp8 score jump")


def test_full_size_workload_sampled_rows():
    """The causal S = 8192 workload (B = 2, H = 32, D = 128) in E4M3, in the
    benchmark's launch configuration; sampled rows of several heads (sequence
    ends, tile and block edges, random rows) against the oracle row by row."""
    w = ai.FP8_WORKLOAD
    bits = ai.make_inputs_fp8(w.B, w.H, w.S, w.D, w.seed)
    rows = P.sample_rows(w.B, w.H, w.S, n_heads=4, n_rows=48, seed=3500, block=256)
    P.check_fp8(bits, w.causal, w.scale, rows_by_head=rows, what="fp8 full size")


def test_full_size_every_unit_written():
    """The same workload with O and LSE starting as NaN: every (head, query
    block) unit of the causal XCD order (heads in groups of four per XCD at
    this size) writes its rows, so nothing stays NaN."""
    import torch
    import exact_attention_128_amd as A
    w = ai.FP8_WORKLOAD
    b8 = ai.make_inputs_fp8(w.B, w.H, w.S, w.D, w.seed)
    dev = torch.device("cuda", 0)
    q, k, v = (ai.to_torch_u8(b8[n], dev) for n in ("q", "k", "v"))
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((w.B, w.H, w.S), float("nan"), dtype=torch.float32, device=dev)
    A.fwd_fp8_out(q, k, v, b8["q_descale"], b8["k_descale"], b8["v_descale"], o, lse,
                  causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())


def test_matrix_core_accumulation_bound():
    """S = 1: the LSE is the single score itself, so its error is the FP8
    matrix core's dot-product error, checked against the contract's
    FP8_EPS * scale * sum_d |q_d k_d| (plus the fp32 bound) on 4096 rows whose
    products span a wide range of magnitudes."""
    B, H, S, D = 1, 4096, 1, 128
    rng = np.random.default_rng(3700)
    bits = {}
    for name in ("q", "k", "v"):
        t = rng.standard_normal((B, H, S, D)) * 2.0 ** rng.integers(-8, 8, (B, H, S, D))
        bits[name], bits[name + "_descale"] = ai.quantize_e4m3(t.astype(np.float32))
    st = P.check_fp8(bits, False, 1.0 / np.sqrt(D), what="fp8 accumulation")
    print("largest LSE error relative to its bound: %.3f" % st["lse_err_over_bound"])


def test_deterministic():
    bits = ai.make_inputs_fp8(2, 4, 777, 128, 3600)
    a = P.gpu_fwd_fp8(bits, True, 0.1)
    b = P.gpu_fwd_fp8(bits, True, 0.1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
