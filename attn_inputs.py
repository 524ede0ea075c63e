"""Seeded synthetic inputs for the attention forward/backward workloads.

Shared by the tests, the benchmark and the smoke check; used on both sides
of every parity comparison (the oracle gets the exact fp64 upcast of the
same bf16 values the GPU gets).  This module holds no attention arithmetic:
only random draws, the fixed input constructions below, and round-to-
nearest-even conversion to bf16.

Recipe (the pages measure on no public dataset; these stand in for the
unspecified FlashAttention-4 forward workload):
  * numpy PCG64, ``default_rng(seed)``, ``standard_normal(dtype=float32)``,
    drawn in the order Q, K, V, dO, each shaped [B,H,S,D];
  * the "rescale stress" construction scales Q and K by 3, sets every
    query's first feature to 4.0 and adds 0.002*j to key j's first feature,
    so each row's running maximum keeps rising along the sequence;
  * everything is rounded to bf16 (round to nearest, ties to even) once,
    after construction.
Very long sequences (hundreds of millions of elements per tensor) use
``make_inputs_chunked``: the same N(0,1) -> bf16 recipe, but each tensor is
cut into a fixed number of row chunks, chunk c of tensor t drawing from its
own PCG64 stream (``SeedSequence(seed).spawn``, child t * chunks + c), so
the chunks can be drawn by parallel threads with a result that does not
depend on the thread count.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np

SEED_BASE = 20260000


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    causal: bool
    stress: bool = False  # rising-maximum construction
    backward: bool = False
    index: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    def describe(self) -> str:
        return "B=%d H=%d S=%d D=%d %s%s%s" % (
            self.B, self.H, self.S, self.D, "causal" if self.causal else "non-causal",
            " rescale-stress" if self.stress else "", " backward" if self.backward else "")


# The five workloads: a tiny one the oracle finishes instantly, a non-causal
# S=2048 forward, two causal long-sequence forwards (one of them built so the
# running maximum keeps rising), and a causal backward.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 128, 64, False, index=1),
    "fwd_s2k": Workload("fwd_s2k", 4, 16, 2048, 128, False, index=2),
    "fwd_causal_s8k": Workload("fwd_causal_s8k", 2, 32, 8192, 128, True, index=3),
    "fwd_stress_s16k": Workload("fwd_stress_s16k", 1, 16, 16384, 128, True, stress=True, index=4),
    "bwd_causal_s4k": Workload("bwd_causal_s4k", 2, 16, 4096, 128, True, backward=True, index=5),
}

# Many short heads: the memory-bound side of the forward's roofline (a few
# flops per byte, so HBM throughput, not the matrix cores, bounds them).  Same
# i.i.d. N(0,1) draws as the five workloads; 2^12 to 2^14 heads each.
SHORT_WORKLOADS = {
    "fwd_short_s128_h4096": Workload("fwd_short_s128_h4096", 64, 64, 128, 128, False, index=6),
    "fwd_short_s64_d64_h8192": Workload("fwd_short_s64_d64_h8192", 128, 64, 64, 64, False,
                                        index=7),
    "fwd_short_s32_causal_h16384": Workload("fwd_short_s32_causal_h16384", 256, 64, 32, 128,
                                            True, index=8),
}

# every named workload, by name
ALL_WORKLOADS = {**WORKLOADS, **SHORT_WORKLOADS}

# The FP8 forward measured on the causal long-sequence shape (same seed and
# draws as fwd_causal_s8k, quantized to E4M3 per tensor).
FP8_WORKLOAD = Workload("fwd_causal_s8k_fp8", 2, 32, 8192, 128, True, index=3)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, nearest-even; returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x7FFF + lsb wraps in 32 bits only for NaN patterns, replaced below
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to fp64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def make_inputs(B: int, H: int, S: int, D: int, seed: int, stress: bool = False,
                with_dout: bool = False) -> dict:
    """Draw Q, K, V (and dO) as bf16 bit arrays [B,H,S,D] (uint16)."""
    rng = np.random.default_rng(seed)
    shape = (B, H, S, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if stress:
        q *= np.float32(3.0)
        k *= np.float32(3.0)
        q[..., 0] = np.float32(4.0)
        k[..., 0] += (np.float32(0.002) * np.arange(S, dtype=np.float32))[None, None, :]
    out = {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v)}
    del q, k, v
    if with_dout:
        out["do"] = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    return out


def make_inputs_chunked(B: int, H: int, S: int, D: int, seed: int, with_dout: bool = False,
                        chunks: int = 64, threads: int | None = None) -> dict:
    """Q, K, V (and dO) as bf16 bit arrays [B,H,S,D], N(0,1), drawn chunk-wise
    from independent streams (see the module docstring)."""
    names = ["q", "k", "v"] + (["do"] if with_dout else [])
    rows = B * H * S
    bounds = [rows * c // chunks for c in range(chunks + 1)]
    children = np.random.SeedSequence(seed).spawn(len(names) * chunks)
    out = {n: np.empty((rows, D), dtype=np.uint16) for n in names}
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))

    def fill(task):
        t, c = divmod(task, chunks)
        r0, r1 = bounds[c], bounds[c + 1]
        rng = np.random.Generator(np.random.PCG64(children[task]))
        x = rng.standard_normal((r1 - r0, D), dtype=np.float32)
        out[names[t]][r0:r1] = f32_to_bf16_bits(x)

    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, range(len(names) * chunks)))
    return {n: a.reshape(B, H, S, D) for n, a in out.items()}


# ---- FP8 (OCP E4M3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
#      infinities, 0x7f / 0xff are NaN, largest finite 448) for the FP8 forward.

E4M3_MAX = 448.0


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to E4M3, nearest-even; returns uint8 codes.  The
    caller keeps |x| <= 448 (the format has no infinities)."""
    x = np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    if not np.all(np.isfinite(a)) or a.max(initial=0.0) > E4M3_MAX:
        raise ValueError("E4M3 input outside [-448, 448]")
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                # unbiased exponent, subnormals share -6
    q = np.rint(np.ldexp(a, 3 - e))           # significand in units of 2^(e-3), ties to even
    up = q >= 16                              # rounded up into the next binade
    e = np.where(up, e + 1, e)
    q = np.where(up, q / 2, q)
    normal = q >= 8
    code = np.where(normal, ((e + 7) << 3) + (q - 8), q).astype(np.int64)
    code = np.where(a == 0, 0, code)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def e4m3_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact value of E4M3 codes (NaN for 0x7f / 0xff)."""
    b = np.ascontiguousarray(b, dtype=np.uint8).astype(np.int64)
    E, m = (b >> 3) & 15, b & 7
    v = np.where(E == 0, np.ldexp(m.astype(np.float64), -9),
                 np.ldexp((8 + m).astype(np.float64), E - 10))
    v = np.where((E == 15) & (m == 7), np.nan, v)
    return np.where(b & 0x80, -v, v)


def quantize_e4m3(x: np.ndarray):
    """Per-tensor scaling to E4M3 (the largest magnitude maps to at most 448):
    returns (codes uint8, descale float) with x ~= descale * value(codes)."""
    amax = float(np.abs(x).max(initial=0.0))
    descale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    while amax / float(descale) > E4M3_MAX:
        descale = np.nextafter(descale, np.float32(np.inf))
    return f32_to_e4m3_bits((x.astype(np.float64) / float(descale)).astype(np.float32)), float(descale)


def make_inputs_fp8(B: int, H: int, S: int, D: int, seed: int, stress: bool = False) -> dict:
    """Q, K, V drawn exactly as make_inputs (fp32, before any rounding), then
    each quantized to E4M3 with its own per-tensor descale factor:
    {"q", "k", "v": uint8 codes [B,H,S,D], "q_descale", "k_descale", "v_descale"}.
    The exact values are descale * e4m3_bits_to_f64(codes)."""
    rng = np.random.default_rng(seed)
    shape = (B, H, S, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if stress:
        q *= np.float32(3.0)
        k *= np.float32(3.0)
        q[..., 0] = np.float32(4.0)
        k[..., 0] += (np.float32(0.002) * np.arange(S, dtype=np.float32))[None, None, :]
    out = {}
    for name, t in (("q", q), ("k", k), ("v", v)):
        out[name], out[name + "_descale"] = quantize_e4m3(t)
    return out


def fp8_dequantized(bits: dict) -> dict:
    """fp64 values of an FP8 input set (exact: 4-bit significands times an
    fp32 descale)."""
    return {n: e4m3_bits_to_f64(bits[n]) * bits[n + "_descale"] for n in ("q", "k", "v")}


def to_torch_u8(codes: np.ndarray, device=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.to(device) if device is not None else t


def workload_inputs(w: Workload) -> dict:
    return make_inputs(w.B, w.H, w.S, w.D, w.seed, stress=w.stress, with_dout=w.backward)


def to_torch_bf16(bits: np.ndarray, device=None):
    """View uint16 bf16 bit patterns as a torch.bfloat16 tensor (copied to device)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t


def torch_bf16_to_bits(t) -> np.ndarray:
    """Bit patterns of a torch.bfloat16 tensor as a uint16 numpy array."""
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
