"""The forward and backward captured in a HIP graph (torch.cuda.graph) and
replayed: every launch goes on the caller's stream and the library makes no
allocation, copy, memset or synchronisation, so a captured step recomputes
exactly what the eager calls compute.  Each replay is checked bit for bit
against eager calls on the same inputs, with eager work and synchronisations
between replays and new inputs copied into the captured buffers."""
import numpy as np
import pytest

import attn_inputs as ai

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _same(a, b):
    import torch
    return torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("noalloc", [True, False])
def test_captured_step_matches_eager(noalloc):
    import torch
    import exact_attention_128_amd as A
    B, H, S, D, causal = 2, 3, 700, 128, True
    scale = 1.0 / np.sqrt(D)
    dev = torch.device("cuda", 0)
    sets = [ai.make_inputs(B, H, S, D, 5100 + i, with_dout=True) for i in range(3)]
    q, k, v, do = (ai.to_torch_bf16(sets[0][n], dev) for n in ("q", "k", "v", "do"))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    ws = torch.empty(A.bwd_workspace_size(B, H, S, D), dtype=torch.uint8, device=dev)

    def step():
        A.fwd_out(q, k, v, o, lse, causal=causal, scale=scale)
        if noalloc:
            A.bwd_noalloc_out(q, k, v, o, lse, do, dq, dk, dv, causal=causal, scale=scale)
        else:
            A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal, scale=scale)

    def eager(bits):
        tq, tk, tv, tdo = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
        eo, el = A.fwd(tq, tk, tv, causal=causal, scale=scale)
        edq, edk, edv = A.bwd(tq, tk, tv, eo, el, tdo, causal=causal, scale=scale)
        torch.cuda.synchronize()
        return eo, el, edq, edk, edv

    # warm-up outside capture (library load, per-device lookups), then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(5):
        bits = sets[rep % len(sets)]
        for n, t in (("q", q), ("k", k), ("v", v), ("do", do)):
            t.copy_(ai.to_torch_bf16(bits[n], dev))
        for t in (o, dq, dk, dv, lse):
            t.fill_(float("nan"))   # eager work between replays; stale results would show
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager(bits)
        for name, got, want in zip(("O", "LSE", "dQ", "dK", "dV"), (o, lse, dq, dk, dv), ref):
            assert _same(got, want), "replay %d: %s differs from the eager call" % (rep, name)
        print("replay", rep, "bit-identical to eager")
