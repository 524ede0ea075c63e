"""attn_bwd_noalloc (the backward with no workspace argument, on the library's
static per-GPU scratch array) against attn_bwd, the entry point it shares its
kernels with: bit for bit, on two calls in a row, the second with a smaller
problem; plus the host-side rejection of shapes whose statistics exceed the
array (no device touched)."""
import ctypes

import numpy as np
import pytest

import attn_inputs as ai
import parity as P


def test_scratch_limit_rejected_on_the_host():
    import exact_attention_128_amd as A
    lib = A.load()
    cap = lib.attn_noalloc_scratch_bytes()
    assert cap == 32 << 20
    Pp = 0x10000  # fake, aligned: never dereferenced (rejected before any HIP call)
    # 32768 blocks of 64 rows (1 KiB each) fill the array exactly; one more row
    # block is too many
    B, H, D = 1, 32, 128
    for S, want in ((65536 + 1, 9), (1 << 20, 9)):
        assert lib.attn_bwd_workspace_size(B, H, S, D) > cap
        rc = lib.attn_bwd_noalloc(Pp, Pp, Pp, Pp, Pp, Pp, Pp, Pp, Pp, B, H, S, D, 0.1, 1, None)
        assert rc == want
    assert lib.attn_bwd_workspace_size(B, H, 65536, D) == cap
    # the other checks come first, as in attn_bwd
    assert lib.attn_bwd_noalloc(None, Pp, Pp, Pp, Pp, Pp, Pp, Pp, Pp, 1, 1, 16, 128, 0.1, 1,
                                None) == 1
    assert lib.attn_bwd_noalloc(Pp, Pp, Pp, Pp, Pp, Pp, Pp, Pp, Pp, 1, 1, 16, 96, 0.1, 1,
                                None) == 3
    assert lib.attn_strerror(9).decode().startswith("problem needs more scratch")


@pytest.mark.gpu
def test_noalloc_matches_attn_bwd_twice():
    import torch
    import exact_attention_128_amd as A
    dev = torch.device("cuda", 0)
    for (B, H, S, D, causal, seed) in ((2, 4, 1100, 128, True, 71), (1, 3, 300, 64, False, 72)):
        print("case", B, H, S, D, causal, flush=True)
        bits = ai.make_inputs(B, H, S, D, seed, with_dout=True)
        scale = 1.0 / np.sqrt(D)
        q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
        o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
        ref = A.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
        got = [torch.full_like(q, float("nan")) for _ in range(3)]
        A.bwd_noalloc_out(q, k, v, o, lse, do, *got, causal=causal, scale=scale)
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g.view(torch.int16), r.view(torch.int16)), \
                "%s differs from attn_bwd (B=%d H=%d S=%d D=%d)" % (name, B, H, S, D)
        # and both within the stated bound of the oracle
        gd = tuple(ai.bf16_bits_to_f64(ai.torch_bf16_to_bits(t)) for t in got)
        oref = P.oracle_bwd_heads(bits, causal, scale, range(B * H))
        oref = tuple(np.stack([oref[hd][i] for hd in range(B * H)]).reshape(B, H, S, D)
                     for i in range(3))
        P.assert_grads_ok(P.grad_errors(gd, oref), "noalloc B=%d H=%d S=%d" % (B, H, S))
