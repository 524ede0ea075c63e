"""GPU parity of the HIP forward against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest

import attn_inputs as ai
import parity as P

pytestmark = pytest.mark.gpu


def _full_case(B, H, S, D, causal, seed, scale=None, stress=False, rescale_log2=None):
    bits = ai.make_inputs(B, H, S, D, seed, stress=stress)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    o, lse, _ = P.gpu_fwd(bits, causal, scale, rescale_log2)
    o_ref, lse_ref = P.oracle_fwd_full(bits, causal, scale)
    return P.fwd_errors(o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_workload(causal):
    w = ai.WORKLOADS["tiny"]
    bits = ai.workload_inputs(w)
    o, lse, _ = P.gpu_fwd(bits, causal, w.scale)
    o_ref, lse_ref = P.oracle_fwd_full(bits, causal, w.scale)
    P.assert_fwd_ok(P.fwd_errors(o, lse, o_ref, lse_ref), "tiny causal=%s" % causal)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 17, 64, 128, 130, 256, 257, 1000])
def test_ragged_lengths(S, D, causal):
    """S <= 128 runs the one-pass short-sequence kernel; S = 130, 256 and 257
    take the long-sequence kernel's first (partial) steps."""
    err = _full_case(1, 3, S, D, causal, seed=1000 + S + D + int(causal))
    P.assert_fwd_ok(err, "S=%d D=%d causal=%s" % (S, D, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_short_sequence_many_blocks(causal):
    """Short-sequence kernel with many workgroups: 150 heads of 100 rows (one
    128-row block each, the last 28 rows idle), every element against the
    oracle."""
    err = _full_case(3, 50, 100, 128, causal, seed=2001 + int(causal))
    P.assert_fwd_ok(err, "short many blocks causal=%s" % causal)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,heads", [(1, 5), (9, 7), (32, 6), (33, 3), (50, 9), (64, 5), (65, 3)])
def test_short_sequence_packed_heads(S, heads, D, causal):
    """Heads packed per workgroup: four heads of <= 32 rows, or two of <= 64
    rows, per workgroup.  Head counts that leave one to three slots of the
    last workgroup empty, every element against the oracle."""
    err = _full_case(1, heads, S, D, causal, seed=2100 + S + heads + D + int(causal))
    P.assert_fwd_ok(err, "packed S=%d heads=%d D=%d causal=%s" % (S, heads, D, causal))


@pytest.mark.parametrize("S", [24, 64])
def test_short_sequence_packed_many_heads(S):
    """Many packed workgroups: 2001 heads (not a multiple of 2 or 4), every
    element against the oracle."""
    err = _full_case(3, 667, S, 128, True, seed=2200 + S)
    P.assert_fwd_ok(err, "packed many heads S=%d" % S)


def test_short_sequence_counting_makes_no_tests():
    """At S <= 128 the counting entry runs the one-pass kernel, which makes no
    rescale test: zero events, and the same bits as attn_fwd_ex."""
    import torch
    import exact_attention_128_amd as A
    bits = ai.make_inputs(2, 3, 120, 128, 2002, stress=True)
    dev = torch.device("cuda", 0)
    q, k, v = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v"))
    o, lse, tests, resc = A.fwd_rescale_events(q, k, v, causal=True, scale=0.09, rescale_log2=0.0)
    o2, lse2 = A.fwd(q, k, v, causal=True, scale=0.09, rescale_log2=0.0)
    torch.cuda.synchronize()
    assert tests == 0 and resc == 0
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)


@pytest.mark.parametrize("causal", [False, True])
def test_many_heads(causal):
    # 320 heads: the grid is several times the CU count, and B*H is not a
    # multiple of 8 on one side (plain block order) and is on the other.
    err = _full_case(2, 160, 200, 128, causal, seed=77)
    P.assert_fwd_ok(err, "many heads")
    err = _full_case(3, 5, 300, 64, causal, seed=78)
    P.assert_fwd_ok(err, "odd heads")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_multi_block_lengths(D, causal):
    """Several 256-row query blocks and 128-key steps with a ragged tail, and
    B*H = 8, which takes the XCD-aware block order."""
    err = _full_case(2, 4, 1500, D, causal, seed=1500 + D + int(causal))
    P.assert_fwd_ok(err, "S=1500 D=%d causal=%s" % (D, causal))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(3, 67, 600, 128), (1, 40, 3000, 128), (2, 9, 1111, 64)])
def test_many_units(shape, causal):
    """Grids of several workgroups per CU in both block orders: 201 heads of 3
    query blocks (plain order, 603 workgroups), 40 heads of 12 blocks (XCD
    order, 480 workgroups), 18 heads of 5 blocks at D = 64; every element
    against the oracle."""
    B, H, S, D = shape
    err = _full_case(B, H, S, D, causal, seed=4000 + S + int(causal))
    P.assert_fwd_ok(err, "persistent %s causal=%s" % (shape, causal))


@pytest.mark.parametrize("shape", [(1, 48, 4096, 128), (1, 72, 4096, 128), (1, 64, 8192, 64)])
def test_causal_head_groups(shape):
    """The causal XCD order in K/V-sized head groups: 6 heads per XCD in
    groups of 3 (S = 4096, 2 MiB of K/V per head), 9 per XCD with no divisor
    that fits (all at once), 8 per XCD in groups of 4 at D = 64.  One row of
    every 256-row query block of every head, plus the block edges, against
    the oracle, so a block computed twice, never, or for the wrong head
    shows."""
    B, H, S, D = shape
    bits = ai.make_inputs(B, H, S, D, 4100 + H + D)
    scale = 1.0 / np.sqrt(D)
    o, lse, _ = P.gpu_fwd(bits, True, scale)
    rows = {}
    for hd in range(B * H):
        r = {0, 255, 256, S // 2, S - 1}
        r.update(256 * b + (37 * b + 11 * hd) % 256 for b in range(S // 256))
        rows[hd] = np.array(sorted(r), dtype=np.int64)
    err = P.sampled_fwd_errors(o, lse, bits, True, scale, rows)
    print(shape, err)
    P.assert_fwd_ok(err, "head groups %s" % (shape,))


@pytest.mark.parametrize("scale", [1.0, -0.09, 0.0, 0.5, 16.0])
def test_scale_values(scale):
    """Off-standard scales, up to 16 (scores of a few hundred, rows dominated by
    one or two keys: far inside the fp32 range the header requires)."""
    for causal in (False, True):
        err = _full_case(1, 2, 190, 128, causal, seed=90, scale=scale)
        P.assert_fwd_ok(err, "scale=%g causal=%s" % (scale, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_rising_maximum_d64(causal):
    """The rising-maximum construction at D = 64 (the S = 16384 workload is D = 128)."""
    err = _full_case(1, 3, 2100, 64, causal, seed=64, stress=True)
    P.assert_fwd_ok(err, "rising maximum D=64 causal=%s" % causal)


def test_rescale_threshold_gives_same_result():
    """Conditional rescaling is exact: every threshold matches the oracle.  Runs with
    different thresholds use different stale maxima, so P is rounded to bf16 at
    different points: each normalised weight carries a relative rounding error of at
    most 2^-8 (P and l), hence two runs differ by at most 2 * 2^-8 * max|V| plus the
    output rounding (1 ulp each)."""
    bits = ai.make_inputs(1, 4, 3000, 128, 44, stress=True)
    scale = 1.0 / np.sqrt(128)
    o_ref, lse_ref = P.oracle_fwd_full(bits, True, scale)
    vmax = np.abs(ai.bf16_bits_to_f64(bits["v"])).max(axis=(2, 3), keepdims=True)
    outs = {}
    for tau in (0.0, 8.0, 20.0, 32.0, 64.0):
        o, lse, _ = P.gpu_fwd(bits, True, scale, rescale_log2=tau)
        P.assert_fwd_ok(P.fwd_errors(o, lse, o_ref, lse_ref), "tau=%g" % tau)
        outs[tau] = o
    for tau in (8.0, 20.0, 32.0, 64.0):
        diff = np.abs(outs[tau] - outs[0.0])
        bound = 2 * 2.0 ** -8 * vmax + 2 * P.bf16_ulp(o_ref)
        assert np.all(diff <= bound), "tau=%g vs 0: max diff %.3e" % (tau, diff.max())


@pytest.mark.parametrize("poly", [4, 8])
def test_exp_policies_match_oracle(poly):
    """FA4's polynomial exp2 for every 4th / 8th exponential: the same result as
    the hardware exponential, against the oracle, at several thresholds (the
    rising-maximum input rescales often at low thresholds, so the polynomial
    also runs on the rescale path) and at D = 64 non-causal."""
    bits = ai.make_inputs(1, 4, 3000, 128, 45, stress=True)
    scale = 1.0 / np.sqrt(128)
    o_ref, lse_ref = P.oracle_fwd_full(bits, True, scale)
    for tau in (0.0, 8.0, 32.0):
        o, lse, _ = P.gpu_fwd(bits, True, scale, rescale_log2=tau, exp_poly_every=poly)
        P.assert_fwd_ok(P.fwd_errors(o, lse, o_ref, lse_ref), "poly=%d tau=%g" % (poly, tau))
    bits = ai.make_inputs(2, 3, 1500, 64, 46)
    o, lse, _ = P.gpu_fwd(bits, False, 0.125, exp_poly_every=poly)
    o_ref, lse_ref = P.oracle_fwd_full(bits, False, 0.125)
    P.assert_fwd_ok(P.fwd_errors(o, lse, o_ref, lse_ref), "poly=%d D=64" % poly)


def test_default_policy_is_the_one_attn_fwd_runs():
    """attn_fwd gives the same bits as attn_fwd_policy with the policy that
    attn_fwd_default_policy reports for the shape."""
    import exact_attention_128_amd as A
    bits = ai.make_inputs(1, 2, 700, 128, 47)
    tau, poly = A.default_policy(128, True, 700)
    _, l1, b1 = P.gpu_fwd(bits, True, 0.1)
    _, l2, b2 = P.gpu_fwd(bits, True, 0.1, rescale_log2=tau, exp_poly_every=poly)
    assert np.array_equal(b1, b2) and np.array_equal(l1, l2)


def _expected_tests(B, H, S, causal):
    """Rescale tests the kernel makes: one per wave (32 query rows) and 128-key
    step after the wave's first step."""
    n = 0
    for qw in range(0, S, 32):
        wend = min(S, qw + 32) if causal else S
        n += max(0, -(-wend // 128) - 1)
    return B * H * n


@pytest.mark.parametrize("name", ["fwd_stress_s16k", "fwd_causal_s8k", "fwd_s2k"])
def test_rescale_event_counts(name):
    """The counting forward gives attn_fwd_ex's outputs bit for bit, makes exactly
    the number of rescale tests the shape implies, and fires fewer rescales at a
    higher threshold.  On unit-variance scores no later score exceeds the stale
    maximum by more than ~8 nats (under 2^12 per weight), so a lane's 64 weights
    stay far below 2^32 and tau = 32 never fires there."""
    import torch
    import exact_attention_128_amd as A
    w = ai.WORKLOADS[name]
    bits = ai.workload_inputs(w)
    dev = torch.device("cuda", 0)
    q, k, v = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v"))
    fired = {}
    for tau in (0.0, 8.0, 32.0):
        o, lse, tests, resc = A.fwd_rescale_events(q, k, v, causal=w.causal, scale=w.scale,
                                                   rescale_log2=tau)
        o2, lse2 = A.fwd(q, k, v, causal=w.causal, scale=w.scale, rescale_log2=tau)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "O differs at tau=%g" % tau
        assert torch.equal(lse, lse2), "LSE differs at tau=%g" % tau
        assert tests == _expected_tests(w.B, w.H, w.S, w.causal), (tests, tau)
        fired[tau] = resc
        print(name, "tau", tau, "tests", tests, "rescales", resc,
              "(%.2f%%)" % (100.0 * resc / max(1, tests)))
    assert fired[0.0] >= fired[8.0] >= fired[32.0]
    if not w.stress:
        assert fired[32.0] == 0


def test_deterministic():
    bits = ai.make_inputs(2, 4, 777, 128, 5)
    _, l1, b1 = P.gpu_fwd(bits, True, 0.1)
    _, l2, b2 = P.gpu_fwd(bits, True, 0.1)
    assert np.array_equal(b1, b2) and np.array_equal(l1, l2)


def test_non_default_stream():
    import torch
    bits = ai.make_inputs(1, 8, 513, 128, 6)
    s = torch.cuda.Stream()
    o, lse, _ = P.gpu_fwd(bits, False, 1.0 / np.sqrt(128), stream=s)
    o_ref, lse_ref = P.oracle_fwd_full(bits, False, 1.0 / np.sqrt(128))
    P.assert_fwd_ok(P.fwd_errors(o, lse, o_ref, lse_ref), "side stream")


@pytest.mark.parametrize("name", ["fwd_s2k", "fwd_causal_s8k", "fwd_stress_s16k",
                                  *ai.SHORT_WORKLOADS])
def test_full_size_workloads(name):
    """Full-size workloads in the benchmark's launch configuration, every element
    of O and LSE against the oracle (about 10 s of oracle time each for the two
    long causal ones), including the many-head short-sequence workloads."""
    w = ai.ALL_WORKLOADS[name]
    bits = ai.workload_inputs(w)
    o, lse, _ = P.gpu_fwd(bits, w.causal, w.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o_ref, lse_ref = P.oracle_fwd_full(bits, w.causal, w.scale)
    err = P.fwd_errors(o, lse, o_ref, lse_ref)
    print(name, err)
    P.assert_fwd_ok(err, name)
    if w.stress:
        # the other softmax policy corner on the same oracle: FA4's threshold 8
        # with every 4th exponential by the polynomial
        o, lse, _ = P.gpu_fwd(bits, w.causal, w.scale, rescale_log2=8.0, exp_poly_every=4)
        err = P.fwd_errors(o, lse, o_ref, lse_ref)
        print(name, "tau 8, poly 4", err)
        P.assert_fwd_ok(err, name + " tau 8 poly 4")


@pytest.mark.parametrize("causal", [False, True])
def test_large_score_jump(causal):
    """A late key whose score exceeds every earlier score by ~150 nats (over 128
    in log2 units), so the weights computed against the stale row maximum
    overflow to inf and the rescale path must recover from the kept exponents.
    Queries are 2u and key 600 is 7u for one random sign vector u (exact in
    bf16); every other key is N(0,1)."""
    B, H, S, D = 1, 2, 700, 128
    bits = ai.make_inputs(B, H, S, D, 4242)
    rng = np.random.default_rng(4243)
    u = np.where(rng.random(D) < 0.5, -1.0, 1.0).astype(np.float32)
    q = np.broadcast_to(2.0 * u, (B, H, S, D))
    k = ai.bf16_bits_to_f32(bits["k"]).copy()
    k[:, :, 600, :] = 7.0 * u
    bits["q"] = ai.f32_to_bf16_bits(q)
    bits["k"] = ai.f32_to_bf16_bits(k)
    scale = 1.0 / np.sqrt(D)
    o, lse, _ = P.gpu_fwd(bits, causal, scale)
    o_ref, lse_ref = P.oracle_fwd_full(bits, causal, scale)
    assert lse_ref.max() > 150.0
    P.assert_fwd_ok(P.fwd_errors(o, lse, o_ref, lse_ref), "score jump causal=%s" % causal)
