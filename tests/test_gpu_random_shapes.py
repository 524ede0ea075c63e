"""Seeded random shapes against the oracle: forward and backward over draws of
(B, H, S, D, causal, scale) that reach every size-dependent path -- the short
kernel's three packings, the long kernel's ragged first and last steps, both
block orders (B*H a multiple of 8 or not), and the backward's partial key and
query blocks.  Small enough for the oracle to check every element."""
import numpy as np
import pytest

import attn_inputs as ai
import parity as P

pytestmark = pytest.mark.gpu

N_CASES = 24


def _cases():
    rng = np.random.default_rng(20260601)
    out = []
    for i in range(N_CASES):
        S = int(rng.choice([int(rng.integers(1, 129)), int(rng.integers(129, 800))]))
        bh = int(rng.choice([8, 16, int(rng.integers(1, 13))]))
        B = int(rng.choice([d for d in (1, 2, 4) if bh % d == 0]))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        scale = float(rng.choice([1.0 / np.sqrt(D), float(rng.uniform(-0.2, 0.2))]))
        out.append((i, B, bh // B, S, D, causal, scale))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "c%d_B%dH%dS%dD%d%s" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else ""))
def test_random_shape(case):
    i, B, H, S, D, causal, scale = case
    print("case", case, flush=True)
    bits = ai.make_inputs(B, H, S, D, 6000 + i, with_dout=True)
    o, lse, _ = P.gpu_fwd(bits, causal, scale)
    o_ref, lse_ref = P.oracle_fwd_full(bits, causal, scale)
    P.assert_fwd_ok(P.fwd_errors(o, lse, o_ref, lse_ref), "random forward %s" % (case,))
    got = P.gpu_fwd_bwd(bits, causal, scale)
    ref = P.oracle_bwd_heads(bits, causal, scale, range(B * H))
    ref = tuple(np.stack([ref[hd][j] for hd in range(B * H)]).reshape(B, H, S, D)
                for j in range(3))
    P.assert_grads_ok(P.grad_errors(got, ref), "random backward %s" % (case,))
