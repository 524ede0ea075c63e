"""GPU parity of the HIP backward (dQ, dK, dV) against the fp64 oracle.

The backward consumes the GPU forward's O and LSE; the oracle recomputes its
own fp64 forward.  Bound: max |err| <= 5e-2 for each gradient."""
import numpy as np
import pytest

import attn_inputs as ai
import oracle
import parity as P

pytestmark = pytest.mark.gpu


def _case(B, H, S, D, causal, seed, scale=None):
    bits = ai.make_inputs(B, H, S, D, seed, with_dout=True)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    got = P.gpu_fwd_bwd(bits, causal, scale)
    ref = P.oracle_bwd_heads(bits, causal, scale, range(B * H))
    ref = tuple(np.stack([ref[hd][i] for hd in range(B * H)]).reshape(B, H, S, D)
                for i in range(3))
    return P.grad_errors(got, ref), got


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 17, 64, 130, 300])
def test_ragged_lengths(S, D, causal):
    err, _ = _case(1, 2, S, D, causal, seed=2000 + S + D + int(causal))
    P.assert_grads_ok(err, "S=%d D=%d causal=%s" % (S, D, causal))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_multi_block_lengths(D, causal):
    """Several blocks of every kernel (256-row dQ blocks, 128-key dK/dV blocks
    walked in 64-query steps) with ragged tails, and B*H = 8, which takes the
    XCD-aware block order."""
    err, _ = _case(2, 4, 1500, D, causal, seed=2500 + D + int(causal))
    P.assert_grads_ok(err, "S=1500 D=%d causal=%s" % (D, causal))


def _check_scaled_bound(bits, causal, scale, what):
    """Each gradient held to max(5e-2, 2^-7 * max|reference|): two bf16 ulps of
    its largest element (the 5e-2 bound is stated for unit-variance scores)."""
    B, H, S, D = bits["q"].shape
    got = P.gpu_fwd_bwd(bits, causal, scale)
    ref = P.oracle_bwd_heads(bits, causal, scale, range(B * H))
    for i, name in enumerate(("dq", "dk", "dv")):
        r = np.stack([ref[hd][i] for hd in range(B * H)]).reshape(B, H, S, D)
        bound = max(P.GRAD_MAX, 2.0 ** -7 * np.abs(r).max())
        err = np.abs(got[i] - r).max()
        print("%s %s max err %.3e (plain bound %.1e, scaled bound %.3e, max|ref| %.3e)" % (
            what, name, err, P.GRAD_MAX, bound, np.abs(r).max()))
        assert np.isfinite(err) and err <= bound, "%s %s err %.3e > %.3e" % (
            what, name, err, bound)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("scale", [1.0, -0.2, 0.0])
def test_scale_values(scale, D):
    """Off-standard scales.  At scale 1 the gradients reach |dQ| ~ 40, where one
    bf16 ulp of the output alone is 0.25, hence the scaled bound."""
    bits = ai.make_inputs(1, 2, 150, D, 31, with_dout=True)
    _check_scaled_bound(bits, True, scale, "scale=%g D=%d" % (scale, D))


@pytest.mark.parametrize("causal", [False, True])
def test_rising_maximum_inputs(causal):
    """The rising-maximum construction (Q, K scaled by 3, first query feature 4,
    key j's first feature + 0.002 j): scores spread over tens of nats, so most
    probabilities underflow and a few dominate each row."""
    bits = ai.make_inputs(1, 2, 1100, 128, 37, stress=True, with_dout=True)
    _check_scaled_bound(bits, causal, 1.0 / np.sqrt(128), "rising maximum causal=%s" % causal)


def test_deterministic():
    """No atomics anywhere in the backward: two runs on the same inputs give the
    same bits."""
    bits = ai.make_inputs(2, 3, 333, 128, 41, with_dout=True)
    g1 = P.gpu_fwd_bwd(bits, True, 0.1)
    g2 = P.gpu_fwd_bwd(bits, True, 0.1)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


def test_non_default_stream():
    """Forward and backward enqueued on a side stream (the binding launches on
    torch's current stream)."""
    import torch
    import exact_attention_128_amd as A
    B, H, S, D = 1, 4, 257, 128
    bits = ai.make_inputs(B, H, S, D, 42, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    dev = torch.device("cuda", 0)
    q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        o, lse = A.fwd(q, k, v, causal=True, scale=scale)
        dq, dk, dv = A.bwd(q, k, v, o, lse, do, causal=True, scale=scale)
    side.synchronize()
    got = tuple(ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(t)) for t in (dq, dk, dv))
    ref = P.oracle_bwd_heads(bits, True, scale, range(B * H))
    ref = tuple(np.stack([ref[hd][i] for hd in range(B * H)]).reshape(B, H, S, D)
                for i in range(3))
    P.assert_grads_ok(P.grad_errors(got, ref), "side stream")


def test_grid_beyond_16_bits():
    """66 001 heads (B*H not a multiple of 8: plain block order), S = 40, D = 64:
    every kernel's grid exceeds 65 535 workgroups.  Forward and backward,
    every element against the oracle."""
    import torch
    import exact_attention_128_amd as A
    B, H, S, D = 1, 66001, 40, 64
    bits = ai.make_inputs_chunked(B, H, S, D, 61, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    dev = torch.device("cuda", 0)
    q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = A.bwd(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    f64 = {n: ai.bf16_bits_to_f64(bits[n]) for n in bits}
    o_ref, lse_ref = oracle.attn_fwd(f64["q"], f64["k"], f64["v"], scale, True)
    P.assert_fwd_ok(P.fwd_errors(ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(o)),
                                 lse.cpu().numpy().astype(np.float64), o_ref, lse_ref),
                    "66001 heads forward")
    ref = oracle.attn_bwd(f64["q"], f64["k"], f64["v"], f64["do"], scale, True)
    got = tuple(ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(t)) for t in (dq, dk, dv))
    P.assert_grads_ok(P.grad_errors(got, ref), "66001 heads backward")


def test_workspace_contents_do_not_matter():
    """The workspace is filled with NaN bit patterns before the call: every byte
    the kernels read is written by the same call first."""
    import torch
    import exact_attention_128_amd as A
    B, H, S, D = 1, 3, 333, 128
    bits = ai.make_inputs(B, H, S, D, 43, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    dev = torch.device("cuda", 0)
    q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=True, scale=scale)
    ws = torch.full((A.bwd_workspace_size(B, H, S, D),), 0xFF, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=True, scale=scale)
    torch.cuda.synchronize()
    got = tuple(ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(t)) for t in (dq, dk, dv))
    ref = P.oracle_bwd_heads(bits, True, scale, range(B * H))
    ref = tuple(np.stack([ref[hd][i] for hd in range(B * H)]).reshape(B, H, S, D)
                for i in range(3))
    P.assert_grads_ok(P.grad_errors(got, ref), "NaN-filled workspace")


def test_concurrent_calls_on_two_streams():
    """Two host threads enqueue a forward + backward each, of different shapes,
    on two streams at once (the library keeps no state between calls)."""
    import threading
    import torch
    import exact_attention_128_amd as A
    dev = torch.device("cuda", 0)
    cases = [(2, 2, 700, 128, True, 51), (1, 3, 450, 64, False, 52)]
    inputs, results = [], [None, None]
    for (B, H, S, D, causal, seed) in cases:
        bits = ai.make_inputs(B, H, S, D, seed, with_dout=True)
        inputs.append((bits, tuple(ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))))
    torch.cuda.synchronize()

    def work(i):
        B, H, S, D, causal, seed = cases[i]
        q, k, v, do = inputs[i][1]
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            for _ in range(3):
                o, lse = A.fwd(q, k, v, causal=causal)
                grads = A.bwd(q, k, v, o, lse, do, causal=causal)
        st.synchronize()
        results[i] = (o, lse, grads)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i, (B, H, S, D, causal, seed) in enumerate(cases):
        bits = inputs[i][0]
        scale = 1.0 / np.sqrt(D)
        o, lse, grads = results[i]
        o_ref, lse_ref = P.oracle_fwd_full(bits, causal, scale)
        P.assert_fwd_ok(P.fwd_errors(ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(o)),
                                     lse.cpu().numpy().astype(np.float64), o_ref, lse_ref),
                        "thread %d forward" % i)
        got = tuple(ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(t)) for t in grads)
        ref = P.oracle_bwd_heads(bits, causal, scale, range(B * H))
        ref = tuple(np.stack([ref[hd][j] for hd in range(B * H)]).reshape(B, H, S, D)
                    for j in range(3))
        P.assert_grads_ok(P.grad_errors(got, ref), "thread %d backward" % i)


@pytest.mark.parametrize("shape", [(1, 3, 300, 128), (1, 40, 512, 128)])
def test_phase_subsets(shape):
    """attn_bwd_phases: DQ writes the row statistics itself, so DQ then MAIN
    (on a workspace filled with garbage) reproduces the whole backward bit for
    bit; PRE then MAIN gives the same dK, dV up to the summation order of
    Delta, both against the oracle.  The second shape has more padded rows
    than the statistics kernel's grid has lanes (327 680 lanes' worth against
    1024 x 256), so its grid-stride loop runs twice."""
    import torch
    import exact_attention_128_amd as A
    B, H, S, D = shape
    bits = ai.make_inputs(B, H, S, D, 43, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    dev = torch.device("cuda", 0)
    q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=True, scale=scale)
    n = A.bwd_workspace_size(B, H, S, D)

    def run(*phase_list):
        ws = torch.full((n,), 0x7f, dtype=torch.uint8, device=dev)   # garbage
        outs = [torch.full_like(q, float("nan")) for _ in range(3)]
        for ph in phase_list:
            A.bwd_out(q, k, v, o, lse, do, *outs, ws, causal=True, scale=scale, phases=ph)
        torch.cuda.synchronize()
        return [ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(t)) for t in outs]

    full = run(A.BWD_ALL)
    split = run(A.BWD_DQ, A.BWD_MAIN)
    for a_, b_ in zip(full, split):
        assert np.array_equal(a_, b_)
    pre = run(A.BWD_PRE, A.BWD_MAIN)
    ref = P.oracle_bwd_heads(bits, True, scale, range(B * H))
    ref = tuple(np.stack([ref[hd][i] for hd in range(B * H)]).reshape(B, H, S, D)
                for i in range(3))
    err = P.grad_errors((full[0], pre[1], pre[2]), ref)
    P.assert_grads_ok(err, "PRE then MAIN")
    assert np.isnan(pre[0]).all()   # dQ not requested: left untouched


def test_many_heads():
    err, _ = _case(3, 50, 160, 128, True, seed=32)
    P.assert_grads_ok(err, "many heads")


def test_full_size_workload():
    """The causal backward workload (B=2, H=16, S=4096, D=128) in the benchmark's
    launch configuration, every element of every head against the oracle, plus
    an invariant: sum_j dK_j = 0 (each row of dS sums to zero)."""
    w = ai.WORKLOADS["bwd_causal_s4k"]
    bits = ai.workload_inputs(w)
    got = P.gpu_fwd_bwd(bits, w.causal, w.scale)
    for g in got:
        assert np.all(np.isfinite(g))
    heads = list(range(w.B * w.H))
    ref = P.oracle_bwd_heads(bits, w.causal, w.scale, heads)
    for hd in heads:
        b, h = divmod(hd, w.H)
        err = P.grad_errors([g[b, h] for g in got], ref[hd])
        print("head", hd, err)
        P.assert_grads_ok(err, "head %d" % hd)
    colsum = np.abs(got[1].sum(axis=2)).max()
    assert colsum <= 1.0, "sum_j dK_j far from zero: %.3e" % colsum


@pytest.mark.parametrize("phase", ["PRE", "DQ"])
def test_statistics_records(phase):
    """The workspace the dK/dV kernel reads, as both writers leave it (the
    statistics kernel, PRE, and the dQ kernel, DQ): per query row a record of
    three bf16 parts of -LSE*log2(e), three of -Delta, two zeros.  The first
    three parts summed in fp64 and rounded once to fp32 must give back exactly
    the fp32 -LSE*log2(e) (each part is the bf16 rounding of what the earlier
    ones leave, so the rest is below half an fp32 ulp), each part must be
    within half a bf16 ulp of what the earlier ones leave, -Delta must match
    -sum_d dO*O (fp64 on the same bf16 values), and the padding rows of the
    last 64-row block must be all zero."""
    import torch
    import exact_attention_128_amd as A
    B, H, S, D = 2, 3, 300, 128   # 5 blocks of 64 rows, 20 padding rows
    bits = ai.make_inputs(B, H, S, D, 47, with_dout=True)
    dev = torch.device("cuda", 0)
    q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=True, scale=1.0 / np.sqrt(D))
    n = A.bwd_workspace_size(B, H, S, D)
    ws = torch.full((n,), 0x7f, dtype=torch.uint8, device=dev)   # garbage
    outs = [torch.empty_like(q) for _ in range(3)]
    ph = A.BWD_PRE if phase == "PRE" else A.BWD_DQ
    A.bwd_out(q, k, v, o, lse, do, *outs, ws, causal=True, scale=1.0 / np.sqrt(D), phases=ph)
    torch.cuda.synchronize()
    nrows = 64 * ((S + 63) // 64)
    rec = ws.cpu().numpy()[:B * H * nrows * 16].view(np.uint16).reshape(B * H, nrows, 8)
    parts = ai.bf16_bits_to_f64(rec)
    assert np.all(parts[:, S:, :] == 0), "padding rows must be zero"
    assert np.all(rec[:, :, 6:] == 0)
    valid = parts[:, :S, :]
    want_l = (-lse.cpu().numpy().reshape(B * H, S).astype(np.float32)
              * np.float32(1.4426950408889634)).astype(np.float32)
    got_l = (valid[:, :, 0] + valid[:, :, 1] + valid[:, :, 2]).astype(np.float32)
    assert np.array_equal(got_l, want_l), "-LSE*log2(e) not reproduced exactly"
    for j in (0, 3):   # the parts: each the bf16 rounding of what the earlier ones leave
        x = valid[:, :, j] + valid[:, :, j + 1] + valid[:, :, j + 2]
        r1 = x - valid[:, :, j]
        assert np.all(np.abs(r1) <= 2.0 ** -8 * np.abs(x) + 1e-300)
        r2 = r1 - valid[:, :, j + 1]
        assert np.all(np.abs(r2) <= 2.0 ** -8 * np.abs(r1) + 1e-300)
    o64 = ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(o)).reshape(B * H, S, D)
    do64 = ai.bf16_bits_to_f64(bits["do"]).reshape(B * H, S, D)
    want_d = -(o64 * do64).sum(axis=2)
    got_d = valid[:, :, 3] + valid[:, :, 4] + valid[:, :, 5]
    scale_d = (np.abs(o64 * do64)).sum(axis=2) + 1e-30
    assert np.max(np.abs(got_d - want_d) / scale_d) < 1e-6, "-Delta off"


@pytest.mark.parametrize("shape", [(1, 48, 4096, 128), (1, 64, 8192, 64)])
def test_causal_dq_head_groups(shape):
    """The dQ kernel's causal XCD order in K/V-sized head groups (6 heads per
    XCD in groups of 3; 8 per XCD in groups of 4 at D = 64).  A work unit
    reads and writes the rows of the head it is given, so an order that
    computed some (head, query block) twice would leave another never
    computed: dQ starts as NaN and must come out finite everywhere.  The last
    200 query rows of a few heads are checked against the oracle."""
    import torch
    import exact_attention_128_amd as A
    B, H, S, D = shape
    bits = ai.make_inputs(B, H, S, D, 4700 + H + D, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    dev = torch.device("cuda", 0)
    q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=True, scale=scale)
    ws = torch.empty(A.bwd_workspace_size(B, H, S, D), dtype=torch.uint8, device=dev)
    dq = torch.full_like(q, float("nan"))
    dk, dv = torch.empty_like(q), torch.empty_like(q)
    A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=True, scale=scale, phases=A.BWD_DQ)
    torch.cuda.synchronize()
    got = ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(dq))
    assert np.all(np.isfinite(got)), "a (head, query block) of dQ was never computed"
    n = 200
    f64 = {nm: ai.bf16_bits_to_f64(bits[nm]) for nm in ("q", "k", "v", "do")}
    for hd in (0, 7, 8, B * H - 1):
        b, h = divmod(hd, H)
        ref = oracle.attn_bwd_causal_tail(f64["q"][b, h, S - n:], f64["do"][b, h, S - n:],
                                          f64["k"][b, h], f64["v"][b, h], scale)[0]
        err = float(np.abs(got[b, h, S - n:] - ref).max())
        print(shape, "head", hd, "dQ tail max err %.3e" % err)
        assert err <= 5e-2, "head %d dQ tail error %.3e" % (hd, err)
