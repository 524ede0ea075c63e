"""CPU checks behind the FP8 forward's accuracy contract.

* The E4M3 codec of the input generator (attn_inputs) against two outside
  references: PyTorch's CPU float8_e4m3fn cast (every code decoded, random and
  tie values encoded) and the codes the gfx950 conversion instruction
  (v_cvt_pk_fp8_f32) produced for a table of values on the GPU (round to
  nearest even, OCP E4M3, no saturation).
* The per-element bound used by the FP8 parity tests (parity.fp8_row_bounds),
  replayed on emulated kernel arithmetic: weights rounded to E4M3 and O
  normalised by their sum stay inside it on random and peaked rows, while a
  plausible kernel mistake -- normalising by the sum of the unrounded weights,
  or rounding the weights to E4M3 without the 2^2 offset -- leaves it."""
import numpy as np
import pytest

import attn_inputs as ai
import parity as P

# value -> code printed by the GPU conversion instruction
GPU_CODES = [(1.0, 0x38), (1.0625, 0x38), (1.125, 0x39), (1.1875, 0x3A), (448.0, 0x7E),
             (-448.0, 0xFE), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00),
             (1.5 * 2.0 ** -10, 0x01), (2.0 ** -11, 0x00), (0.0, 0x00), (-0.0, 0x80), (3.0, 0x44),
             (0.3, 0x2A), (0.1, 0x1D), (7.5, 0x4F), (256.0, 0x78), (240.0, 0x77),
             (2.0 ** -7, 0x04), (1.09375, 0x39)]


def test_codec_matches_gpu_conversion_table():
    x = np.array([v for v, _ in GPU_CODES], dtype=np.float32)
    want = np.array([c for _, c in GPU_CODES], dtype=np.uint8)
    assert np.array_equal(ai.f32_to_e4m3_bits(x), want)


def test_codec_matches_torch():
    import torch
    allc = np.arange(256, dtype=np.uint8)
    mine = ai.e4m3_bits_to_f64(allc)
    ref = torch.from_numpy(allc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[~np.isnan(mine)], ref[~np.isnan(ref)])
    rng = np.random.default_rng(5)
    x = np.concatenate([np.clip(rng.standard_normal(100000) * 50, -448, 448),
                        (rng.random(20000) * 2.0 ** -5), mine[~np.isnan(mine)]]).astype(np.float32)
    mids = (mine[~np.isnan(mine)][:-1] + np.diff(mine[~np.isnan(mine)]) / 2).astype(np.float32)
    x = np.concatenate([x, mids[np.abs(mids) <= 448]])
    tb = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ai.f32_to_e4m3_bits(x), tb)
    with pytest.raises(ValueError):
        ai.f32_to_e4m3_bits(np.array([449.0], dtype=np.float32))


def test_quantize_uses_the_range():
    x = np.random.default_rng(6).standard_normal((3, 1000)).astype(np.float32)
    codes, ds = ai.quantize_e4m3(x)
    v = ai.e4m3_bits_to_f64(codes)
    assert np.abs(v).max() == 448.0 and ds > 0
    assert np.abs(v * ds - x).max() <= 2.0 ** -4 * np.abs(x).max()


def _emulate(q, k, v, scale, causal, offset=2.0, normalise_rounded=True, score_err=0.0):
    """E4M3 weights as the kernel forms them (scores, each off by up to
    score_err * scale * sum_d |q_d k_d| with a random sign like the FP8 matrix
    core's accumulation, row max, 2^offset offset), O normalised by the rounded
    or the unrounded weights."""
    S = k.shape[0]
    out = np.empty_like(q)
    rng = np.random.default_rng(9)
    for i in range(S):
        nv = i + 1 if causal else S
        s = scale * (k[:nv] @ q[i])
        s = s + score_err * scale * (np.abs(k[:nv]) @ np.abs(q[i])) * rng.choice([-1.0, 1.0], nv)
        e = (2.0 ** offset) * np.exp(s - s.max())
        er = ai.e4m3_bits_to_f64(ai.f32_to_e4m3_bits(e.astype(np.float32)))
        out[i] = (er @ v[:nv]) / (er.sum() if normalise_rounded else e.sum())
    return out


def _ratio(q, k, v, scale, causal, o):
    import oracle
    o_ref, _ = oracle.attn_fwd(q[None, None], k[None, None], v[None, None], scale, causal)
    o_ref = o_ref[0, 0]
    b = P.fp8_row_bounds(q, k, v, scale, causal, np.arange(q.shape[0]), o_ref)
    return float((np.abs(o - o_ref) / b).max())


@pytest.mark.parametrize("case", ["unit", "peaked"])
def test_bound_holds_for_the_kernel_arithmetic_and_catches_mistakes(case):
    rng = np.random.default_rng(7 if case == "unit" else 8)
    S, D = 300, 64
    sc = 1.0 if case == "unit" else 6.0
    q, k, v = (ai.e4m3_bits_to_f64(ai.f32_to_e4m3_bits(
        np.clip(rng.standard_normal((S, D)) * f, -448, 448).astype(np.float32)))
        for f in (sc, sc, 1.0))
    scale = 1.0 / np.sqrt(D)
    for causal in (False, True):
        good = _ratio(q, k, v, scale, causal, _emulate(q, k, v, scale, causal))
        assert good <= 1.0, (case, causal, good)
        # the matrix core's score error at the contract's full allowance
        good = _ratio(q, k, v, scale, causal, _emulate(q, k, v, scale, causal,
                                                       score_err=P.FP8_EPS))
        assert good <= 1.0, (case, causal, good)
    if case == "peaked":
        bad = _ratio(q, k, v, scale, True, _emulate(q, k, v, scale, True, normalise_rounded=False))
        assert not bad <= 1.0, bad
    else:
        # no headroom: the largest weight at E4M3's smallest normal, the rest subnormal
        with np.errstate(invalid="ignore"):
            bad = _ratio(q, k, v, scale, False, _emulate(q, k, v, scale, False, offset=-6.0))
        assert not bad <= 1.0, bad
