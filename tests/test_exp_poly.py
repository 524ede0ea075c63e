"""The forward kernel's software exponential, FA4's polynomial exp2 on the FMA
pipe (Tencent Cloud article "AI Infra 系列 第六章 GPU 性能工程（二）", section 7):
2^x = 2^n * p(f) with n = floor(x), f = x - n in [0, 1) and p a cubic.  The
coefficients are read from the kernel source and the kernel's fp32 steps
(clamp, floor, three FMAs, ldexp) are replayed in numpy, each rounded to fp32,
then pinned against fp64 exp2:
  * relative error <= 1e-4 over a dense sweep of f in [0, 1) and of x in
    [-126, 64] (the bf16 rounding that P undergoes next is 2^-9 ~ 2e-3);
  * p(0) = 1 exactly, so every integer x gives the exact power of two;
  * x = -inf (a masked key) and x <= -160 give exactly 0.
A planted mistake in the coefficients (a dropped term, a wrong sign) fails."""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "exact_attention_128_amd", "csrc", "attn_fwd.hip")


def _coeffs():
    text = open(SRC).read()
    vals = {}
    for name in ("kExpP1", "kExpP2", "kExpP3"):
        m = re.search(r"constexpr float %s = ([0-9.eE+-]+)f;" % name, text)
        assert m, "%s not found in attn_fwd.hip" % name
        vals[name] = np.float32(float(m.group(1)))
    clamp = re.search(r"fmaxf\(x, (-[0-9.]+)f\)", text)
    assert clamp, "clamp of the exponent argument not found"
    return vals["kExpP1"], vals["kExpP2"], vals["kExpP3"], np.float32(float(clamp.group(1)))


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def exp2_poly(x, p1, p2, p3, lo):
    """The kernel's steps in fp32 (each FMA rounded once: the exact product of
    two fp32 values plus an fp32 addend, rounded from fp64)."""
    x = np.maximum(_f32(x), lo)
    n = np.floor(x)
    f = _f32(x.astype(np.float64) - n)
    p = _f32(p3.astype(np.float64) * f + p2)
    p = _f32(p.astype(np.float64) * f + p1)
    p = _f32(p.astype(np.float64) * f + 1.0)
    with np.errstate(over="ignore", under="ignore"):
        return np.ldexp(p, n.astype(np.int64).clip(-1000, 1000)).astype(np.float32)


def check(p1, p2, p3, lo):
    f = _f32(np.linspace(0.0, 1.0, 1 << 20, endpoint=False))
    got = exp2_poly(f, p1, p2, p3, lo).astype(np.float64)
    rel = np.max(np.abs(got / np.exp2(f.astype(np.float64)) - 1.0))
    assert rel <= 1e-4, "relative error on [0,1): %.3e" % rel
    x = _f32(np.linspace(-126.0, 64.0, 1 << 20))
    got = exp2_poly(x, p1, p2, p3, lo).astype(np.float64)
    rel = np.max(np.abs(got / np.exp2(x.astype(np.float64)) - 1.0))
    assert rel <= 1e-4, "relative error on [-126, 64]: %.3e" % rel
    ints = np.arange(-126, 65, dtype=np.float32)
    assert np.array_equal(exp2_poly(ints, p1, p2, p3, lo), np.exp2(ints).astype(np.float32))
    assert np.all(exp2_poly(np.array([-np.inf, -160.0, -1e30], dtype=np.float32), p1, p2, p3,
                            lo) == 0.0)
    return rel


def test_kernel_polynomial_meets_its_bound():
    p1, p2, p3, lo = _coeffs()
    rel = check(p1, p2, p3, lo)
    print("max relative error %.3e" % rel)


@pytest.mark.parametrize("mutant", ["drop_cubic", "sign", "swap"])
def test_bound_catches_planted_mistakes(mutant):
    p1, p2, p3, lo = _coeffs()
    if mutant == "drop_cubic":
        p3 = np.float32(0.0)
    elif mutant == "sign":
        p2 = -p2
    else:
        p1, p2 = p2, p1
    with pytest.raises(AssertionError):
        check(p1, p2, p3, lo)
