"""The fp64 oracle against its pins, and the pins against planted mistakes.

Every pin in oracle_pins.py must pass on the real oracle.  Then each entry of
MUTANTS plants one plausible mistake in a private copy of oracle.c (a wrong
causal bound, a dropped scale, a wrong sign, a swapped operand, ...), compiles
it, and requires that at least one pin fails, so no pin set is vacuous.
"""
import os

import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.default())


def test_thread_count_does_not_change_results():
    orc = oracle.default()
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 2, 70, 16)) for _ in range(3))
    n0 = orc.max_threads()
    try:
        orc.set_threads(1)
        a = orc.attn_fwd(q, k, v, 0.3, True)
        orc.set_threads(max(2, n0))
        b = orc.attn_fwd(q, k, v, 0.3, True)
    finally:
        orc.set_threads(n0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# (name, text in oracle.c, replacement, how many occurrences to replace (0 = all))
MUTANTS = [
    ("causal_excludes_diagonal", "return causal ? pos + 1 : S;", "return causal ? pos : S;", 1),
    ("scale_dropped", "s_buf[j] = scale * dot;", "s_buf[j] = dot;", 1),
    ("no_max_subtraction", "s_buf[j] = exp(s_buf[j] - m);", "s_buf[j] = exp(s_buf[j]);", 1),
    ("lse_without_max", "*lse = m + log(l);", "*lse = log(l);", 1),
    ("unnormalised_o", "const double p = s_buf[j] / l;", "const double p = s_buf[j];", 1),
    ("values_reversed", "o[d] += p * v[j * D + d];", "o[d] += p * v[(n - 1 - j) * D + d];", 1),
    ("keys_reversed", "for (long d = 0; d < D; ++d) dot += q[d] * k[j * D + d];",
     "for (long d = 0; d < D; ++d) dot += q[d] * k[(n - 1 - j) * D + d];", 1),
    ("ds_wrong_sign", "p * (dp - delta[i])", "p * (dp + delta[i])", 0),
    ("dk_scale_dropped", "for (long d = 0; d < D; ++d) dkj[d] *= scale;", "", 1),
    ("dq_scale_dropped", "for (long d = 0; d < D; ++d) dqi[d] *= scale;", "", 1),
    ("dv_uses_ds", "dvj[d] += p * doi[d];", "dvj[d] += ds * doi[d];", 1),
    ("dq_uses_values", "dqi[d] += ds * k[j * D + d];", "dqi[d] += ds * v[j * D + d];", 1),
    ("dk_causal_off_by_one", "const long i0 = causal ? j : 0;",
     "const long i0 = causal ? j + 1 : 0;", 1),
    ("delta_from_dout_only", "dl += doi[d] * o[i * D + d];", "dl += doi[d] * doi[d];", 1),
    ("dk_uses_dout", "dkj[d] += ds * qi[d];", "dkj[d] += ds * doi[d];", 1),
    ("tail_dq_skips_diagonal", "for (long j = 0; j <= i; ++j) {", "for (long j = 0; j < i; ++j) {",
     1),
    ("tail_dkdv_skips_diagonal", "for (long r = c; r < n; ++r) {",
     "for (long r = c + 1; r < n; ++r) {", 1),
    ("tail_p_scale_dropped", "const double p = exp(scale * dot - lse[r]);",
     "const double p = exp(dot - lse[r]);", 0),
    ("batched_head_offset", "const long off = hd * S * D;", "const long off = hd * S;", 1),
    ("batched_causal_dropped", "scale, causal, dq + off", "scale, 0, dq + off", 1),
    ("batched_first_batch_only", "for (long hd = 0; hd < B * H; ++hd) {",
     "for (long hd = 0; hd < H; ++hd) {", 1),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant, tmp_path):
    name, old, new, count = mutant
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert old in src, "mutation target missing: %r" % old
    src = src.replace(old, new) if count == 0 else src.replace(old, new, count)
    path = tmp_path / ("oracle_%s.c" % name)
    path.write_text(src)
    lib = oracle.compile_source(str(path), str(tmp_path / ("lib_%s.so" % name)))
    bad = oracle.Oracle(lib)
    failures = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(bad)
            except (AssertionError, RuntimeError, FloatingPointError, ValueError) as e:
                failures.append(pin.__name__)
    assert failures, "no pin caught the planted mistake %s" % name
