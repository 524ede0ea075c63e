"""Seeded random-shape parity sweep, longer than the committed GPU tests (not
collected by pytest; run it by name on a machine with a GPU):

    python tests/sweep_random_shapes.py --seed 4242 --cases 500 --max-s 2600
    python tests/sweep_random_shapes.py --fp8 --seed 31337 --cases 150

bf16: forward and backward of each drawn (B, H, S, D, causal, scale), every
element against the oracle, with the bounds of tests/parity.py (the plain
gradient bound, not the two-ulp bound of the off-workload tests, so cases with
large gradients show up as outliers to inspect).  --fp8: the FP8 forward
against its bound.  Prints one line per case and a summary; exit status 1 if
any case failed."""
import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402

import attn_inputs as ai  # noqa: E402
import parity as P  # noqa: E402


def draw(rng, max_s, max_scale):
    S = int(rng.choice([int(rng.integers(1, 140)), int(rng.integers(140, max_s))]))
    bh = int(rng.choice([8, 16, 24, int(rng.integers(1, 13))]))
    B = int(rng.choice([d for d in (1, 2, 4) if bh % d == 0]))
    D = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    scale = float(rng.choice([1.0 / np.sqrt(D), float(rng.uniform(-max_scale, max_scale))]))
    return B, bh // B, S, D, causal, scale


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seed", type=int, default=4242)
    ap.add_argument("--cases", type=int, default=100)
    ap.add_argument("--max-s", type=int, default=2600)
    ap.add_argument("--max-scale", type=float, default=0.25)
    ap.add_argument("--fp8", action="store_true")
    a = ap.parse_args()
    rng = np.random.default_rng(a.seed)
    fails, t0 = 0, time.time()
    for i in range(a.cases):
        B, H, S, D, causal, scale = draw(rng, a.max_s, a.max_scale)
        case = (i, B, H, S, D, causal, scale)
        try:
            if a.fp8:
                P.check_fp8(ai.make_inputs_fp8(B, H, S, D, a.seed + i), causal, scale,
                            what="fp8 %s" % (case,))
            else:
                bits = ai.make_inputs(B, H, S, D, a.seed + i, with_dout=True)
                o, lse, _ = P.gpu_fwd(bits, causal, scale)
                o_ref, lse_ref = P.oracle_fwd_full(bits, causal, scale)
                P.assert_fwd_ok(P.fwd_errors(o, lse, o_ref, lse_ref), "forward %s" % (case,))
                got = P.gpu_fwd_bwd(bits, causal, scale)
                ref = P.oracle_bwd_heads(bits, causal, scale, range(B * H))
                ref = tuple(np.stack([ref[hd][j] for hd in range(B * H)]).reshape(B, H, S, D)
                            for j in range(3))
                err = P.grad_errors(got, ref)
                big = max(float(np.abs(r).max()) for r in ref)
                try:
                    P.assert_grads_ok(err, "backward %s" % (case,))
                except AssertionError as e:
                    raise AssertionError("%s; largest reference element %.3f, bf16 ulp there %.4f"
                                         % (e, big, float(P.bf16_ulp(big))))
            print("ok", case, "%.0fs" % (time.time() - t0), flush=True)
        except AssertionError as e:
            fails += 1
            print("FAIL", case, e, flush=True)
    print("done: %d cases, %d failures" % (a.cases, fails), flush=True)
    return 1 if fails else 0


if __name__ == "__main__":
    sys.exit(main())
