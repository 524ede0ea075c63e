"""Pins that tie the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` instance and raises
AssertionError when the oracle disagrees with:
  * hand-derived closed-form cases (tests/golden/closed_form_cases.json);
  * closed forms of softmax attention (constant V, causal row 0, zero Q);
  * invariances (a shift added to every key, a joint permutation of the
    key/value rows);
  * an independent brute-force evaluation in 50-digit arithmetic (mpmath)
    with no maximum subtraction;
  * PyTorch's CPU fp64 scaled_dot_product_attention and autograd;
  * central finite differences of L = sum(dO * O) for the backward;
  * backward invariants (sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, causal
    dQ_0 = 0, constant V gives dQ = dK = 0).
The same functions run against deliberately broken copies of the oracle
(test_oracle.py) to show that each plausible mistake trips at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "closed_form_cases.json")


def _val(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"log": math.log}))  # own fixture file
    return float(x)


def _arr(rows):
    return np.array([[_val(x) for x in r] for r in rows], dtype=np.float64)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    if not np.all(np.isfinite(a)):
        raise AssertionError("%s: non-finite values" % what)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, "%s: max abs err %.3e > %.1e" % (what, err, tol)


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- forward pins

def pin_golden_forward(orc):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q, k, v = _arr(c["q"]), _arr(c["k"]), _arr(c["v"])
        for mode in ("noncausal", "causal"):
            if mode not in c:
                continue
            causal = mode == "causal"
            exp_o, exp_lse = _arr(c[mode]["o"]), np.array([_val(x) for x in c[mode]["lse"]])
            if c.get("rows_only"):
                pos = np.full(q.shape[0], k.shape[0] - 1)
                o, lse = orc.attn_fwd_rows(q, pos, k, v, c["scale"], causal)
            else:
                o, lse = orc.attn_fwd(q[None, None], k[None, None], v[None, None], c["scale"],
                                      causal)
                o, lse = o[0, 0], lse[0, 0]
            _close(o, exp_o, 1e-12, "%s/%s O" % (c["name"], mode))
            _close(lse, exp_lse, 1e-12, "%s/%s LSE" % (c["name"], mode))


def pin_golden_backward(orc):
    cases = json.load(open(GOLDEN))["cases"]
    n = 0
    for c in cases:
        if "backward_noncausal" not in c:
            continue
        g = c["backward_noncausal"]
        q, k, v, do = _arr(c["q"]), _arr(c["k"]), _arr(c["v"]), _arr(g["dout"])
        dq, dk, dv, _, _ = orc.attn_bwd_head(q, k, v, do, c["scale"], False)
        _close(dq, _arr(g["dq"]), 1e-12, c["name"] + " dQ")
        _close(dk, _arr(g["dk"]), 1e-12, c["name"] + " dK")
        _close(dv, _arr(g["dv"]), 1e-12, c["name"] + " dV")
        n += 1
    assert n > 0


def pin_constant_v(orc):
    """V_j = u for every j  =>  O_i = u (the probabilities of a row sum to 1)."""
    rng = np.random.default_rng(11)
    B, H, S, D = 2, 2, 37, 8
    q, k = _rand(rng, B, H, S, D, scale=2.0), _rand(rng, B, H, S, D, scale=2.0)
    u = _rand(rng, B, H, 1, D)
    v = np.broadcast_to(u, (B, H, S, D)).copy()
    for causal in (False, True):
        o, _ = orc.attn_fwd(q, k, v, 0.35, causal)
        _close(o, np.broadcast_to(u, o.shape), 1e-12, "constant V causal=%s" % causal)


def pin_rows_of_p(orc):
    """V = identity (S = D, V_j = e_j) makes O_i the probability row P_i itself:
    each row is nonnegative and sums to 1, P_ij = exp(s_ij - LSE_i) for every
    visible key, and causal rows put no weight above the diagonal."""
    rng = np.random.default_rng(14)
    S = D = 16
    q, k = _rand(rng, 1, 1, S, D, scale=1.5), _rand(rng, 1, 1, S, D, scale=1.5)
    v = np.eye(S)[None, None]
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, 0.4, causal)
        p, lse = o[0, 0], lse[0, 0]
        assert np.all(p >= 0.0), "negative probability causal=%s" % causal
        _close(p.sum(axis=1), np.ones(S), 1e-12, "rows of P sum to 1 causal=%s" % causal)
        s = 0.4 * q[0, 0] @ k[0, 0].T
        vis = np.tril(np.ones((S, S), dtype=bool)) if causal else np.ones((S, S), dtype=bool)
        want = np.where(vis, np.exp(s - lse[:, None]), 0.0)
        _close(p, want, 1e-12, "P_ij = exp(s_ij - LSE_i) causal=%s" % causal)


def pin_causal_row0(orc):
    """Causal row 0 sees key 0 only: O_0 = V_0, LSE_0 = scale * q_0 . k_0."""
    rng = np.random.default_rng(12)
    B, H, S, D = 1, 3, 19, 16
    q, k, v = (_rand(rng, B, H, S, D) for _ in range(3))
    o, lse = orc.attn_fwd(q, k, v, 0.25, True)
    _close(o[:, :, 0], v[:, :, 0], 1e-12, "causal row 0 O")
    _close(lse[:, :, 0], 0.25 * np.sum(q[:, :, 0] * k[:, :, 0], -1), 1e-12, "causal row 0 LSE")


def pin_zero_q(orc):
    """Q = 0: uniform weights, O_i = mean of the visible V_j, LSE_i = ln(#visible)."""
    rng = np.random.default_rng(13)
    B, H, S, D = 1, 2, 23, 8
    q = np.zeros((B, H, S, D))
    k, v = _rand(rng, B, H, S, D), _rand(rng, B, H, S, D)
    o, lse = orc.attn_fwd(q, k, v, 1.0, False)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), 1e-12, "zero Q O")
    _close(lse, np.full(lse.shape, math.log(S)), 1e-12, "zero Q LSE")
    o, lse = orc.attn_fwd(q, k, v, 1.0, True)
    cnt = np.arange(1, S + 1, dtype=np.float64)
    _close(o, np.cumsum(v, axis=2) / cnt[None, None, :, None], 1e-12, "zero Q causal O")
    _close(lse, np.broadcast_to(np.log(cnt), lse.shape), 1e-12, "zero Q causal LSE")


def pin_key_shift(orc):
    """K_j += u for all j: O unchanged, LSE_i += scale * q_i . u."""
    rng = np.random.default_rng(14)
    B, H, S, D = 1, 2, 29, 8
    q, k, v = (_rand(rng, B, H, S, D) for _ in range(3))
    u = _rand(rng, D)
    for causal in (False, True):
        o1, l1 = orc.attn_fwd(q, k, v, 0.4, causal)
        o2, l2 = orc.attn_fwd(q, k + u, v, 0.4, causal)
        _close(o2, o1, 1e-11, "key shift O causal=%s" % causal)
        _close(l2, l1 + 0.4 * (q @ u), 1e-11, "key shift LSE causal=%s" % causal)


def pin_permutation(orc):
    """A joint permutation of the key and value rows leaves a non-causal result unchanged,
    while permuting the values alone changes it."""
    rng = np.random.default_rng(15)
    B, H, S, D = 1, 1, 31, 8
    q, k, v = (_rand(rng, B, H, S, D) for _ in range(3))
    perm = rng.permutation(S)
    o1, l1 = orc.attn_fwd(q, k, v, 0.5, False)
    o2, l2 = orc.attn_fwd(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    _close(o2, o1, 1e-12, "joint permutation O")
    _close(l2, l1, 1e-12, "joint permutation LSE")
    o3, _ = orc.attn_fwd(q, k, v[:, :, perm], 0.5, False)
    assert np.max(np.abs(o3 - o1)) > 1e-3, "values-only permutation should change O"


def pin_mpmath_bruteforce(orc):
    """S <= 16: direct 50-digit evaluation without max subtraction."""
    import mpmath
    mpmath.mp.dps = 50
    rng = np.random.default_rng(16)
    for (S, D, causal, scale) in ((1, 4, False, 0.5), (5, 3, True, 1.0), (16, 8, False, 0.3),
                                  (16, 8, True, 0.7), (9, 2, True, 2.0)):
        q, k, v = (_rand(rng, 1, 1, S, D) for _ in range(3))
        o, lse = orc.attn_fwd(q, k, v, scale, causal)
        for i in range(S):
            keys = range(i + 1) if causal else range(S)
            w = [mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(
                mpmath.mpf(q[0, 0, i, d]) * mpmath.mpf(k[0, 0, j, d]) for d in range(D)))
                for j in keys]
            tot = mpmath.fsum(w)
            ref_lse = float(mpmath.log(tot))
            ref_o = [float(mpmath.fsum(w[n] * mpmath.mpf(v[0, 0, j, d]) for n, j in
                                       enumerate(keys)) / tot) for d in range(D)]
            _close(lse[0, 0, i], ref_lse, 1e-12, "mpmath LSE S=%d i=%d" % (S, i))
            _close(o[0, 0, i], ref_o, 1e-12, "mpmath O S=%d i=%d" % (S, i))


def pin_torch_sdpa(orc):
    """PyTorch CPU fp64 scaled_dot_product_attention (library special case)."""
    import torch
    rng = np.random.default_rng(17)
    for (B, H, S, D, causal, scale) in ((2, 3, 33, 16, False, 0.25), (1, 2, 47, 8, True, 0.35),
                                        (1, 1, 64, 64, True, 0.125)):
        q, k, v = (_rand(rng, B, H, S, D) for _ in range(3))
        o, _ = orc.attn_fwd(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                               scale=scale)
        _close(o, ref.numpy(), 1e-12, "torch sdpa S=%d causal=%s" % (S, causal))


def pin_rows_match_full(orc):
    """The sampled-rows entry point agrees with the full forward."""
    rng = np.random.default_rng(18)
    B, H, S, D = 1, 2, 50, 8
    q, k, v = (_rand(rng, B, H, S, D) for _ in range(3))
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, 0.3, causal)
        pos = np.array([0, 7, 19, 49, 3])
        ro, rl = orc.attn_fwd_rows(q[0, 1, pos], pos, k[0, 1], v[0, 1], 0.3, causal)
        _close(ro, o[0, 1, pos], 0.0, "rows vs full O")
        _close(rl, lse[0, 1, pos], 0.0, "rows vs full LSE")


# --------------------------------------------------------------- backward pins

def _loss(orc, q, k, v, do, scale, causal):
    o, _ = orc.attn_fwd(q[None, None], k[None, None], v[None, None], scale, causal)
    return float(np.sum(o[0, 0] * do))


def pin_finite_differences(orc):
    """Central differences of L = sum(dO * O) match dQ, dK, dV (relative error <= 1e-6)."""
    rng = np.random.default_rng(19)
    h = 1e-6
    for (S, D, causal, scale) in ((6, 4, False, 0.5), (7, 3, True, 0.8)):
        q, k, v, do = (_rand(rng, S, D) for _ in range(4))
        dq, dk, dv, _, _ = orc.attn_bwd_head(q, k, v, do, scale, causal)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args = {"q": q, "k": k, "v": v}
                args[name] = xp
                lp = _loss(orc, args["q"], args["k"], args["v"], do, scale, causal)
                args[name] = xm
                lm = _loss(orc, args["q"], args["k"], args["v"], do, scale, causal)
                num[idx] = (lp - lm) / (2 * h)
            rel = np.max(np.abs(num - g)) / max(1e-300, np.max(np.abs(num)))
            assert rel <= 1e-6, "finite differences d%s causal=%s rel err %.2e" % (name, causal,
                                                                                  rel)


def pin_torch_autograd(orc):
    """PyTorch CPU fp64 autograd through scaled_dot_product_attention."""
    import torch
    rng = np.random.default_rng(20)
    for (S, D, causal, scale) in ((33, 16, True, 0.25), (40, 8, False, 0.4)):
        q, k, v, do = (_rand(rng, S, D) for _ in range(4))
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                               is_causal=causal, scale=scale)
        out.backward(torch.from_numpy(do)[None])
        dq, dk, dv, o, _ = orc.attn_bwd_head(q, k, v, do, scale, causal)
        _close(o, out.detach().numpy()[0], 1e-12, "autograd O")
        _close(dq, tq.grad.numpy(), 1e-11, "autograd dQ causal=%s" % causal)
        _close(dk, tk.grad.numpy(), 1e-11, "autograd dK causal=%s" % causal)
        _close(dv, tv.grad.numpy(), 1e-11, "autograd dV causal=%s" % causal)


def pin_causal_tail_autograd(orc):
    """The causal tail backward (last n rows' dQ, last n keys' dK/dV) against
    PyTorch CPU fp64 autograd of the whole head, sliced to those rows/keys;
    n = S covers the whole head, n = 1 the last position alone."""
    import torch
    rng = np.random.default_rng(22)
    S, D, scale = 37, 8, 0.35
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                           is_causal=True, scale=scale)
    out.backward(torch.from_numpy(do)[None])
    for n in (1, 11, S):
        dq, dk, dv = orc.attn_bwd_causal_tail(q[S - n:], do[S - n:], k, v, scale)
        _close(dq, tq.grad.numpy()[S - n:], 1e-11, "tail dQ n=%d" % n)
        _close(dk, tk.grad.numpy()[S - n:], 1e-11, "tail dK n=%d" % n)
        _close(dv, tv.grad.numpy()[S - n:], 1e-11, "tail dV n=%d" % n)


def pin_batched_backward_autograd(orc):
    """The [B,H,S,D] backward (every head of a batch) against PyTorch CPU fp64
    autograd of scaled_dot_product_attention over the same 4-D tensors, causal
    and not.  Each head draws its own values, so a wrong head offset, a head
    skipped, or a causal flag not passed on to the heads shows up."""
    import torch
    rng = np.random.default_rng(23)
    B, H, S, D, scale = 2, 3, 13, 8, 0.45
    q, k, v, do = (_rand(rng, B, H, S, D) for _ in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                               scale=scale)
        out.backward(torch.from_numpy(do))
        dq, dk, dv = orc.attn_bwd(q, k, v, do, scale, causal)
        _close(dq, tq.grad.numpy(), 1e-11, "batched dQ causal=%s" % causal)
        _close(dk, tk.grad.numpy(), 1e-11, "batched dK causal=%s" % causal)
        _close(dv, tv.grad.numpy(), 1e-11, "batched dV causal=%s" % causal)


def pin_backward_invariants(orc):
    rng = np.random.default_rng(21)
    S, D = 24, 8
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv, _, _ = orc.attn_bwd_head(q, k, v, do, 0.5, causal)
        # sum_j dS_ij = 0 for every row  =>  sum_j dK_j = 0
        _close(dk.sum(0), np.zeros(D), 1e-11, "sum dK causal=%s" % causal)
        # sum_j P_ij = 1  =>  sum_j dV_j = sum_i dO_i
        _close(dv.sum(0), do.sum(0), 1e-11, "sum dV causal=%s" % causal)
        if causal:
            _close(dq[0], np.zeros(D), 1e-12, "causal dQ_0")
    # constant V: O does not depend on Q or K
    vc = np.broadcast_to(_rand(rng, 1, D), (S, D)).copy()
    dq, dk, _, _, _ = orc.attn_bwd_head(q, k, vc, do, 0.5, True)
    _close(dq, np.zeros_like(dq), 1e-11, "constant V dQ")
    _close(dk, np.zeros_like(dk), 1e-11, "constant V dK")


FORWARD_PINS = [pin_golden_forward, pin_constant_v, pin_rows_of_p, pin_causal_row0, pin_zero_q, pin_key_shift,
                pin_permutation, pin_mpmath_bruteforce, pin_torch_sdpa, pin_rows_match_full]
BACKWARD_PINS = [pin_golden_backward, pin_finite_differences, pin_torch_autograd,
                 pin_causal_tail_autograd, pin_batched_backward_autograd, pin_backward_invariants]
ALL_PINS = FORWARD_PINS + BACKWARD_PINS
