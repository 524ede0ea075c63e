"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the fp64 oracle on the same bf16 inputs, and compare element by element.

Tolerances (bf16 inputs, fp32 accumulation): O max |err| <= 2e-2 and mean
|err| <= 2e-3, LSE max |err| <= 1e-3, dQ/dK/dV max |err| <= 5e-2.
"""
from __future__ import annotations

import numpy as np

import attn_inputs as ai
import oracle

O_MAX, O_MEAN, LSE_MAX, GRAD_MAX = 2e-2, 2e-3, 1e-3, 5e-2


def gpu_fwd(bits, causal, scale, rescale_log2=None, stream=None, exp_poly_every=None):
    """Run the forward on cuda:0; returns (O as fp64 numpy, LSE fp64 numpy, O bits)."""
    import torch
    import exact_attention_128_amd as A
    dev = torch.device("cuda", 0)
    q, k, v = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v"))
    kw = dict(causal=causal, scale=scale, rescale_log2=rescale_log2, exp_poly_every=exp_poly_every)
    if stream is None:
        o, lse = A.fwd(q, k, v, **kw)
    else:
        with torch.cuda.stream(stream):
            o, lse = A.fwd(q, k, v, **kw)
        stream.synchronize()
    torch.cuda.synchronize()
    ob = ai.torch_bf16_to_bits(o)
    return ai.bf16_bits_to_f64(ob), lse.cpu().numpy().astype(np.float64), ob


def oracle_fwd_full(bits, causal, scale):
    q, k, v = (ai.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v"))
    return oracle.attn_fwd(q, k, v, scale, causal)


def sample_rows(B, H, S, n_heads, n_rows, seed, block=128):
    """Pick heads and rows: sequence start/end, tile and block edges, random rows."""
    rng = np.random.default_rng(seed)
    heads = sorted(set([0, B * H - 1] + list(rng.choice(B * H, size=min(n_heads, B * H),
                                                          replace=False))))[:max(2, n_heads)]
    fixed = [0, 1, 31, 32, 63, 64, block - 1, block, S // 2, S - 2, S - 1]
    out = {}
    for hd in heads:
        rows = set(r for r in fixed if 0 <= r < S)
        rows.update(rng.choice(S, size=min(n_rows, S), replace=False).tolist())
        out[hd] = np.array(sorted(rows), dtype=np.int64)
    return out


def oracle_fwd_rows(bits, causal, scale, rows_by_head):
    """Oracle O/LSE for the sampled rows: {head: (O [n,D], LSE [n])}."""
    B, H, S, D = bits["q"].shape
    q = bits["q"].reshape(B * H, S, D)
    k = bits["k"].reshape(B * H, S, D)
    v = bits["v"].reshape(B * H, S, D)
    res = {}
    for hd, rows in rows_by_head.items():
        res[hd] = oracle.attn_fwd_rows(ai.bf16_bits_to_f64(q[hd, rows]), rows,
                                       ai.bf16_bits_to_f64(k[hd]), ai.bf16_bits_to_f64(v[hd]),
                                       scale, causal)
    return res


def fwd_errors(o, lse, o_ref, lse_ref):
    do = np.abs(o - o_ref)
    dl = np.abs(lse - lse_ref)
    return {"o_max": float(do.max()), "o_mean": float(do.mean()), "lse_max": float(dl.max())}


def assert_fwd_ok(err, what=""):
    assert np.isfinite(err["o_max"]) and np.isfinite(err["lse_max"]), "%s non-finite %s" % (what,
                                                                                             err)
    assert err["o_max"] <= O_MAX, "%s O max err %.3e > %.1e (%s)" % (what, err["o_max"], O_MAX,
                                                                     err)
    assert err["o_mean"] <= O_MEAN, "%s O mean err %.3e > %.1e" % (what, err["o_mean"], O_MEAN)
    assert err["lse_max"] <= LSE_MAX, "%s LSE err %.3e > %.1e" % (what, err["lse_max"], LSE_MAX)


def sampled_fwd_errors(o, lse, bits, causal, scale, rows_by_head):
    B, H, S, D = bits["q"].shape
    ref = oracle_fwd_rows(bits, causal, scale, rows_by_head)
    o = o.reshape(B * H, S, D)
    lse = lse.reshape(B * H, S)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for hd, rows in rows_by_head.items():
        got_o.append(o[hd, rows])
        got_l.append(lse[hd, rows])
        ref_o.append(ref[hd][0])
        ref_l.append(ref[hd][1])
    return fwd_errors(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o),
                      np.concatenate(ref_l))


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (2^(e-7)); smallest normal spacing for 0."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def gpu_fwd_bwd(bits, causal, scale):
    """Forward then backward on cuda:0 (the backward consumes the GPU forward's O
    and LSE).  Returns fp64 numpy (dQ, dK, dV)."""
    import torch
    import exact_attention_128_amd as A
    dev = torch.device("cuda", 0)
    q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
    o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = A.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return tuple(ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(t)) for t in (dq, dk, dv))


def oracle_bwd_heads(bits, causal, scale, heads):
    """Oracle (dQ, dK, dV) for the listed heads of a [B,H,S,D] problem."""
    B, H, S, D = bits["q"].shape
    arr = {n: bits[n].reshape(B * H, S, D) for n in ("q", "k", "v", "do")}
    out = {}
    for hd in heads:
        dq, dk, dv, _, _ = oracle.attn_bwd_head(*(ai.bf16_bits_to_f64(arr[n][hd])
                                                  for n in ("q", "k", "v", "do")), scale, causal)
        out[hd] = (dq, dk, dv)
    return out


def grad_errors(got, ref):
    return {n: float(np.max(np.abs(g - r))) for n, g, r in zip(("dq", "dk", "dv"), got, ref)}


def assert_grads_ok(err, what=""):
    for n, e in err.items():
        assert np.isfinite(e) and e <= GRAD_MAX, "%s %s max err %.3e > %.1e (%s)" % (
            what, n, e, GRAD_MAX, err)


# ---- FP8 forward: the bound of its accuracy contract (E4M3 weights).
#
# The kernel rounds each softmax weight (offset so that a row's largest weight
# in the first tile is 4) to E4M3 before the PV product and normalises by the
# sum of the rounded weights, so O is a convex combination of V rows with
# perturbed weights.  With e_j = 4 exp(s_j - max s) (the frame in which the
# row's largest weight is exactly 4; the kernel's stale-maximum frame only
# scales all weights up, which can only shrink the relative rounding error),
# each rounded weight is within d_j = 2^-4 e_j + min(e_j, 2^-10) of e_j (half an
# ulp relative for normal E4M3 values, half the subnormal spacing 2^-9
# absolute below them, and flushed-to-zero weights losing at most themselves),
# hence per element
#   |O_i - O_ref_i| <= sum_j d_j |V_j - O_ref_i| / (sum_j e_j - sum_j d_j)
# plus the bf16 output rounding (2^-9 relative, taken as 2^-8 for the fp32
# normalisation) and the fp32 accumulation over up to 2^13 keys (1e-3 max|V|).
#
# The scores themselves carry the FP8 matrix core's accumulation error: it
# does not add its 64 exact products in full fp32 (measured on gfx950:
# |err| <= 2^-11.6 sum_k |a_k b_k| with widely mixed magnitudes, 2^-14.7 for
# N(0,1) operands), so each score is within FP8_EPS * A_ij of exact, with
# A_ij = |scale| sum_d |Q_id K_jd| and FP8_EPS = 2^-10 (a margin of 3 over the
# worst measured).  A weight is then perturbed by a factor within
# exp(+-FP8_EPS A_ij) before its E4M3 rounding, and the LSE (a smooth maximum
# of the scores) by at most max_j FP8_EPS A_ij on top of the fp32 bound 1e-3.
FP8_U = 2.0 ** -4
FP8_FLUSH = 2.0 ** -10
FP8_EPS = 2.0 ** -10


def fp8_row_bounds(q, k, v, scale, causal, rows, o_ref, with_lse=False):
    """Per-element bounds [n, D] for query rows `rows` of one head (fp64
    inputs [S, D], o_ref the oracle's O for those rows [n, D]); with
    with_lse, also the per-row LSE bounds [n]."""
    S = k.shape[0]
    out = np.empty_like(o_ref)
    lse_b = np.empty(len(rows))
    ak = np.abs(k)
    for n, i in enumerate(rows):
        nv = i + 1 if causal else S
        s = scale * (k[:nv] @ q[i])
        a = abs(scale) * (ak[:nv] @ np.abs(q[i]))
        e = 4.0 * np.exp(s - s.max())
        d = ((1.0 + FP8_U) * np.exp(FP8_EPS * a) - 1.0) * e + np.minimum(e, FP8_FLUSH)
        dev = np.abs(v[:nv] - o_ref[n][None, :])
        out[n] = (d @ dev) / (e.sum() - d.sum()) + 2.0 ** -8 * np.abs(o_ref[n]) + \
            1e-3 * np.abs(v[:nv]).max()
        lse_b[n] = LSE_MAX + FP8_EPS * a.max()
    return (out, lse_b) if with_lse else out


def gpu_fwd_fp8(bits, causal, scale):
    """FP8 forward on cuda:0; returns (O fp64, LSE fp64)."""
    import torch
    import exact_attention_128_amd as A
    dev = torch.device("cuda", 0)
    q, k, v = (ai.to_torch_u8(bits[n], dev) for n in ("q", "k", "v"))
    o, lse = A.fwd_fp8(q, k, v, bits["q_descale"], bits["k_descale"], bits["v_descale"],
                       causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(o)),
            lse.cpu().numpy().astype(np.float64))


def check_fp8(bits, causal, scale, rows_by_head=None, what=""):
    """FP8 forward against the oracle on the dequantized inputs: every element
    (or the sampled rows) within its bound, LSE within LSE_MAX.  Returns the
    error statistics."""
    B, H, S, D = bits["q"].shape
    o, lse = gpu_fwd_fp8(bits, causal, scale)
    deq = ai.fp8_dequantized(bits)
    qd, kd, vd = (deq[n].reshape(B * H, S, D) for n in ("q", "k", "v"))
    o = o.reshape(B * H, S, D)
    lse = lse.reshape(B * H, S)
    if rows_by_head is None:
        o_ref, lse_ref = oracle.attn_fwd(deq["q"], deq["k"], deq["v"], scale, causal)
        o_ref, lse_ref = o_ref.reshape(B * H, S, D), lse_ref.reshape(B * H, S)
        rows_by_head = {hd: np.arange(S) for hd in range(B * H)}
        ref = {hd: (o_ref[hd], lse_ref[hd]) for hd in rows_by_head}
    else:
        ref = {hd: oracle.attn_fwd_rows(qd[hd, rows], rows, kd[hd], vd[hd], scale, causal)
               for hd, rows in rows_by_head.items()}
    worst, errs, lerr, lworst = 0.0, [], 0.0, 0.0
    for hd, rows in rows_by_head.items():
        r_o, r_l = ref[hd]
        got = o[hd, rows]
        bound, lbound = fp8_row_bounds(qd[hd], kd[hd], vd[hd], scale, causal, rows, r_o,
                                       with_lse=True)
        err = np.abs(got - r_o)
        assert np.all(np.isfinite(got)), "%s non-finite O" % what
        worst = max(worst, float((err / bound).max()))
        errs.append(err)
        le = np.abs(lse[hd, rows] - r_l)
        lerr = max(lerr, float(le.max()))
        lworst = max(lworst, float((le / lbound).max()))
    err = np.concatenate([e.ravel() for e in errs])
    stats = {"o_max": float(err.max()), "o_mean": float(err.mean()),
             "max_err_over_bound": worst, "lse_max": lerr, "lse_err_over_bound": lworst}
    print(what, stats)
    assert worst <= 1.0, "%s O outside its bound: %s" % (what, stats)
    assert lworst <= 1.0, "%s LSE outside its bound: %s" % (what, stats)
    return stats
