#!/usr/bin/env python3
"""Benchmark of the fused exact-attention hot path on one MI355X.

One step = the whole path over one batch of seeded synthetic input: the fused
forward (O, LSE) followed by the backward (dQ with the row statistics, then
dK/dV) that consumes the forward's O and LSE.  The default workload is the
causal backward workload (B=2, H=16, S=4096, D=128, bf16), the one workload
that exercises every step.  Throughput is algorithmic TFLOPS: forward
4*B*H*S^2*D (halved when causal) plus backward 2.5x that, over K timed steps
after W warm-up steps (defaults 100 and 30: the clock settles first).

Also measured, in the same process:
  * the dominant kernel (the backward's dK/dV kernel), timed with HIP events
    on the stream it is launched on, in the same K steps run once more with an
    event between the step's kernels -> "roofline" (MFMA bound); the backward's
    dQ kernel likewise -> "dq_kernel" (each also timed alone, "alone_ms");
  * the forward alone on the four forward workloads (S=128 D=64 non-causal, a
    latency case reported with its algorithmic HBM rate; S=2048 non-causal;
    S=8192 causal; S=16384 causal rising-maximum) -> "legs" and "fwd_roofline";
  * the forward on three many-head short-sequence workloads (S=128, 64, 32),
    bound by HBM, each with its algorithmic HBM rate -> "legs" and
    "short_roofline" (HBM bound, S=128);
  * the FP8 (E4M3) forward on the S=8192 causal shape against the FP8 peak;
  * calibration legs that are not on the path: a library bf16 GEMM (what the
    matrix cores sustain) and a 1 GiB device copy (what HBM sustains);
  * the forward and the whole backward each alone, back to back -> "fwd_ms",
    "bwd_ms";
  * from rocprofv3 records of the same kernel sources (reported only while
    the sources' digest matches): HBM bytes per launch -> "traffic", and wall
    cycles per launch -> "cycles_profiled", "frac_at_clock" (work per cycle
    against the peak's) and "step_at_clock" for the whole step;
  * the fp64 CPU oracle on a bounded sample of the same workload on this host's
    cores -> "cpu_baseline" (a reported baseline, not the target).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense FP8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch of the dominant kernel (the backward's dK/dV kernel on
# the causal S=4096 workload), from rocprofv3 FETCH_SIZE and WRITE_SIZE runs
# (profiles/bwd_causal_s4k_counters.md), each scaled by what the same counter
# reads for a plain 1 GiB device copy; and the wall cycles of one launch at the
# shader clock in those counter runs (GRBM_GUI_ACTIVE per XCD, mean over the
# passes that hold it).  A compute-bound kernel's cycle count holds far better
# than its clock under the power limit (one run's passes at 1.50-1.60 GHz agree
# to 0.7 %; runs on different boxes to about 3 %), so flops / (peak flops per
# cycle x cycles) is its fraction of the dense peak at the clock it gets, and
# cycles / a live duration estimates the clock of that live run.  Valid only for the kernel sources whose digest is
# recorded here; reported as null once they change.
TRAFFIC_SOURCES = ("exact_attention_128_amd/csrc/attn_bwd.hip",
                   "exact_attention_128_amd/csrc/gfx950.h",
                   "exact_attention_128_amd/csrc/attn_internal.h",
                   "exact_attention_128_amd/build.py")
TRAFFIC = {"workload": "bwd_causal_s4k", "read_bytes": 235468705, "write_bytes": 67109173,
           "cycles": 500167,
           "sources_sha256": "9dcb570e1ffcbc2176f3a0c46d72955a4cca3efeb5e094b63396ef7d16258764"}
# the same for the forward on the causal S=8192 workload
# (profiles/fwd_causal_s8k_counters.md)
FWD_TRAFFIC_SOURCES = ("exact_attention_128_amd/csrc/attn_fwd.hip",
                       "exact_attention_128_amd/csrc/gfx950.h",
                       "exact_attention_128_amd/csrc/attn_internal.h",
                       "exact_attention_128_amd/build.py")
FWD_TRAFFIC = {"workload": "fwd_causal_s8k", "read_bytes": 582272535, "write_bytes": 136314880,
               "cycles": 1782431,
               "sources_sha256": "1d7cf01eed59945fef8688b54fc5bc3d679d5caeba268231974cc68888b113e1"}
# the wall cycles of the step's three kernels on the causal S=4096 workload
# (forward, dQ, dK/dV; profiles/bwd_causal_s4k_counters.md): the step's work
# per cycle, whatever clock the power limit leaves it
STEP_SOURCES = ("exact_attention_128_amd/csrc/attn_fwd.hip",
                "exact_attention_128_amd/csrc/attn_bwd.hip",
                "exact_attention_128_amd/csrc/attn_bwd_dq.hip",
                "exact_attention_128_amd/csrc/gfx950.h",
                "exact_attention_128_amd/csrc/attn_internal.h",
                "exact_attention_128_amd/build.py")
STEP_CYCLES = {"workload": "bwd_causal_s4k", "cycles": 285341 + 355852 + 500167,
               "sources_sha256": "3a9824d80ddbaa143b42e9ad0f7db1b2e174c7d7e587832bf01093972d045d70"}


def measured_record(workload, record=None, sources=None):
    """The profiled record of a kernel on a workload, or None when it was taken
    on another workload or the kernel's sources have changed since."""
    import hashlib
    record = TRAFFIC if record is None else record
    sources = TRAFFIC_SOURCES if sources is None else sources
    if workload != record["workload"]:
        return None
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != record["sources_sha256"]:
        return None
    return record


def measured_traffic(workload, record=None, sources=None):
    rec = measured_record(workload, record, sources)
    return None if rec is None else rec["read_bytes"] + rec["write_bytes"]


PEAK_BF16_FLOP_PER_CYCLE = 256 * 4096   # dense bf16 MFMA, whole chip, per shader clock


def at_clock(flops, live_ms, workload, record=None, sources=None):
    """From the profiled cycle count of one launch: {"cycles_profiled",
    "frac_at_clock" = flops / (peak flops per cycle x cycles), the fraction of
    the dense peak at the clock the kernel runs at, and "clock_ghz_live" =
    cycles / the live duration}; all None without a valid record."""
    rec = measured_record(workload, record, sources)
    if rec is None or "cycles" not in rec:
        return {"cycles_profiled": None, "frac_at_clock": None, "clock_ghz_live": None}
    c = rec["cycles"]
    return {"cycles_profiled": c,
            "frac_at_clock": round(flops / (PEAK_BF16_FLOP_PER_CYCLE * c), 4),
            "clock_ghz_live": round(c / (live_ms * 1e-3) / 1e9, 3)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_flops(B, H, S, D, causal):
    f = 4.0 * B * H * S * S * D
    return f / 2 if causal else f


def oracle_fwd_sample(w, bits, budget_s):
    """Time the fp64 oracle's forward on a bounded sample of one forward
    workload: the whole problem when it is small, else chunks of 64 query rows
    spread evenly over the sequence, cycling through the heads, until about
    budget_s of CPU time.  Returns its algorithmic rate (the GPU path's flop
    count for the same rows) and what was sampled."""
    import numpy as np
    import attn_inputs as ai
    import oracle
    B, H, S, D = w.B, w.H, w.S, w.D
    full = fwd_flops(B, H, S, D, w.causal)
    if full <= 1e9:
        f64 = {n: ai.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v")}
        t0 = time.perf_counter()
        oracle.attn_fwd(f64["q"], f64["k"], f64["v"], w.scale, w.causal)
        dt = time.perf_counter() - t0
        return {"tflops": round(full / dt / 1e12, 6), "seconds": round(dt, 3),
                "sample": "whole workload"}
    q, k, v = (bits[n].reshape(B * H, S, D) for n in ("q", "k", "v"))
    n = min(64, S)   # rows per chunk: evenly spaced, distinct
    flops, rows, chunk, t0 = 0.0, 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and rows < B * H * S:
        hd = chunk % (B * H)
        pos = (np.arange(n, dtype=np.int64) * (S // n) + (chunk * 7919) % (S // n)) % S
        oracle.attn_fwd_rows(ai.bf16_bits_to_f64(q[hd, pos]), pos, ai.bf16_bits_to_f64(k[hd]),
                             ai.bf16_bits_to_f64(v[hd]), w.scale, w.causal)
        flops += oracle.rows_flops(pos, S, D, w.causal)
        rows += n
        chunk += 1
    dt = time.perf_counter() - t0
    return {"tflops": round(flops / dt / 1e12, 6), "seconds": round(dt, 3),
            "sample": "%d query rows (%d-row chunks spread over the sequence, %d heads) of %d" % (
                rows, n, min(chunk, B * H), B * H * S)}


def _grids(w):
    """Work-items of each kernel's 1-D grid for workload w (as the library
    launches them), keyed by kernel family."""
    bh, S, D = w.B * w.H, w.S, w.D
    g = {"attn_bwd_dq_kernel": bh * (-(-S // 256)) * 512,
         "attn_bwd_main_kernel": bh * (-(-S // 128)) * 256,
         "attn_bwd_pre_kernel": min(-(-(bh * (-(-S // 64)) * 64 * (D // 8)) // 256), 1024) * 256}
    if w.name.endswith("_fp8"):
        return {"attn_fwd_fp8_kernel": bh * (-(-S // 256)) * 512}
    if S <= 128:
        hpw = 4 if S <= 32 else 2 if S <= 64 else 1   # heads per workgroup
        g["attn_fwd_short_kernel"] = -(-bh // hpw) * 256
    else:
        g["attn_fwd_kernel"] = bh * (-(-S // 256)) * 512
    return g


# share of a workload's algorithmic flops credited to each kernel (the dK/dV
# kernel does four of the backward's five products, the dQ kernel the fifth)
_CREDIT = {"attn_fwd_kernel": ("fwd", 1.0), "attn_fwd_short_kernel": ("fwd", 1.0),
           "attn_fwd_fp8_kernel": ("fwd", 1.0),
           "attn_bwd_main_kernel": ("bwd", 0.8), "attn_bwd_dq_kernel": ("bwd", 0.2)}


def trace_summary(path):
    """Markdown summary of a rocprofv3 kernel-trace CSV (--kernel-trace
    --output-format csv): one row per (kernel, grid size), named by the
    workload whose launch has that grid, with mean / median / min / max
    duration and, for the attention kernels, the algorithmic rate and the
    fraction of the dense peak of the kernel's input type (bf16, or FP8 for
    the E4M3 forward) computed from the trace's mean."""
    import csv
    import statistics
    import attn_inputs as ai
    rows = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = r["Kernel_Name"]
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3   # us
            rows.setdefault((name, int(r["Grid_Size_X"])), []).append(dur)
    total = sum(sum(v) for v in rows.values())
    out = ["| Kernel | Workload | Grid (work-items) | Calls | Mean (us) | Median (us) | Min (us) "
           "| Max (us) | Share | Algorithmic TFLOPS (mean) | Fraction of dense peak "
           "| Algorithmic HBM GB/s (mean, forward) |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for (name, grid), d in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        fam = name.split("<")[0].split("::")[-1].strip()
        targs = name.split("<")[1].split(">")[0].split(",") if "<" in name else []
        wl, tf, frac, gbs = "", "", "", ""
        for w in list(ai.ALL_WORKLOADS.values()) + [ai.FP8_WORKLOAD]:
            if fam.startswith("attn_") and targs and int(targs[0]) == w.D and \
                    (len(targs) < 2 or targs[1].strip() == ("true" if w.causal else "false")) and \
                    _grids(w).get(fam) == grid and (fam.startswith("attn_fwd") or w.backward):
                wl = w.name
                if fam in _CREDIT and (len(targs) < 3 or targs[2].strip() != "true"):
                    kind, share = _CREDIT[fam]
                    f = fwd_flops(w.B, w.H, w.S, w.D, w.causal) * (2.5 if kind == "bwd" else 1.0)
                    t = share * f / (statistics.mean(d) * 1e-6) / 1e12
                    peak = PEAK_FP8_TFLOPS if fam == "attn_fwd_fp8_kernel" else PEAK_BF16_TFLOPS
                    tf, frac = "%.1f" % t, "%.4f of %.1f" % (t / peak, peak)
                    if kind == "fwd":
                        nb = 8.0 * w.B * w.H * w.S * w.D + 4.0 * w.B * w.H * w.S
                        if fam == "attn_fwd_fp8_kernel":   # E4M3 inputs, bf16 O
                            nb -= 3.0 * w.B * w.H * w.S * w.D
                        gbs = "%.1f" % (nb / (statistics.mean(d) * 1e-6) / 1e9)
                break
        shown = name if len(name) <= 100 else name[:60] + " ... (library kernel)"
        out.append("| `%s` | %s | %d | %d | %.1f | %.1f | %.1f | %.1f | %.1f%% | %s | %s | %s |" % (
            shown, wl or "-", grid, len(d), statistics.mean(d), statistics.median(d), min(d),
            max(d), 100.0 * sum(d) / total, tf, frac, gbs))
    return "\n".join(out)


# Counter sets of the hardware-counter profiles, one rocprofv3 run each (one
# run holds at most 8 SQ_, 4 TCC_ and 2 GRBM_ counters); passes 3 and 4 are the
# HBM byte counters, also taken for the calibrating copy.
PMC_PASSES = {
    1: "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_LDS "
       "SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE",
    2: "SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_WAIT_ANY "
       "SQ_WAIT_INST_ANY SQ_INSTS_SALU GRBM_GUI_ACTIVE",
    3: "FETCH_SIZE",
    4: "WRITE_SIZE",
    5: "SQ_LDS_IDX_ACTIVE SQ_LDS_CMD_FIFO_FULL SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_LDS "
       "SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_MISC GRBM_GUI_ACTIVE",
}


def pmc_command(n, workload, outdir):
    """The rocprofv3 command of counter pass n over one workload, writing under
    outdir (run from the repository root)."""
    return ("rocprofv3 --pmc %s --output-format csv -d %s/p%d_%s -o run -- "
            "python3 bench.py --only %s --steps 2 --warmup 1" % (PMC_PASSES[n], outdir, n,
                                                                  workload, workload))


def _pmc_load(path):
    """{kernel name: {counter: mean per-dispatch value}} of one counter CSV,
    plus "_duration_ns": the mean dispatch duration from its timestamps."""
    import csv
    per, dur = {}, {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            k = r["Kernel_Name"]
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if "Start_Timestamp" in r and r["Start_Timestamp"]:
                dur.setdefault(k, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) -
                                                            int(r["Start_Timestamp"]))
    out = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in per.items()}
    for k, d in dur.items():
        out[k]["_duration_ns"] = sum(d.values()) / len(d)
    return out


def _alg_bytes(fam, w):
    """(read, write) algorithmic HBM bytes of one launch of kernel family fam
    on workload w: each input read once and each output written once (bf16
    tensors, E4M3 codes for the FP8 forward's inputs, fp32 LSE and the
    backward's 16-byte statistics record per row, in 64-row blocks)."""
    T = w.B * w.H * w.S * w.D * 2
    L = w.B * w.H * w.S * 4
    ST = w.B * w.H * (-(-w.S // 64)) * 1024
    return {"attn_fwd_kernel": (3 * T, T + L), "attn_fwd_short_kernel": (3 * T, T + L),
            "attn_fwd_fp8_kernel": (3 * T // 2, T + L),
            "attn_bwd_dq_kernel": (5 * T + L, T + ST), "attn_bwd_main_kernel": (4 * T + ST, 2 * T),
            "attn_bwd_pre_kernel": (2 * T + L, ST)}.get(fam, (None, None))


def pmc_summary(root, workload):
    """Markdown summary of the five counter passes of one workload, read from
    <root>/p<n>_<workload>/run_counter_collection.csv, with the HBM byte
    counters scaled by what they read for the 1 GiB calibrating copy
    (<root>/p3_copy, <root>/p4_copy).  Prints per kernel the derived shares,
    the instruction counts, the measured and algorithmic HBM bytes, and every
    raw counter."""
    import os.path as op
    import attn_inputs as ai
    w = ai.FP8_WORKLOAD if workload == ai.FP8_WORKLOAD.name else ai.ALL_WORKLOADS[workload]
    csvf = lambda n, wl: op.join(root, "p%d_%s" % (n, wl), "run_counter_collection.csv")
    copy_kernel = lambda d: next(v for k, v in d.items() if "copyBuffer" in k)
    cf = copy_kernel(_pmc_load(csvf(3, "copy")))["FETCH_SIZE"]
    cw = copy_kernel(_pmc_load(csvf(4, "copy")))["WRITE_SIZE"]
    fs, ws = 1048576.0 / cf, 1048576.0 / cw
    raw, clk = {}, {}
    for n in PMC_PASSES:
        for k, d in _pmc_load(csvf(n, workload)).items():
            if "GRBM_GUI_ACTIVE" in d and "_duration_ns" in d:
                # the clock the kernel ran at in this pass: busy cycles per XCD
                # over the dispatch's duration
                clk.setdefault(k, []).append((d["GRBM_GUI_ACTIVE"] / 8 / d["_duration_ns"],
                                              d["_duration_ns"]))
            d.pop("_duration_ns", None)
            raw.setdefault(k, {}).update(d)
    short = lambda k: k.replace("void ", "").split("(")[0]
    fam = lambda k: short(k).split("<")[0].split("::")[-1]
    kind = "backward after one forward" if w.backward else "forward"
    o = ["# Hardware counters: %s B=%d H=%d S=%d D=%d%s (%s)\n" % (
        workload, w.B, w.H, w.S, w.D, " causal" if w.causal else "", kind),
        "Collected on one MI355X, each counter set in its own run, from the repository root "
        "(the profiler wants `cd /tmp && export TMPDIR=/tmp` first and then absolute paths "
        "to the same files), then summarised by the last command:\n", "```"]
    o += [pmc_command(n, workload, root) for n in PMC_PASSES]
    o += [pmc_command(n, "copy", root) for n in (3, 4)]
    o += ["python3 bench.py --pmc-summary %s %s" % (root, workload), "```\n"]
    o.append("""Values are per dispatch, averaged over the run's dispatches of each kernel.  Derived columns:
- MFMA busy = `SQ_VALU_MFMA_BUSY_CYCLES` / (`GRBM_GUI_ACTIVE` / 8 XCDs x 1024 SIMDs): the share of the
  kernel's wall cycles (at the clock it ran at) in which the matrix cores were busy.
- LDS busy = `SQ_LDS_IDX_ACTIVE` / (`GRBM_GUI_ACTIVE` / 8 x 256 CUs).  Co-exec =
  `SQ_VALU_MFMA_COEXEC_CYCLES` / `SQ_VALU_MFMA_BUSY_CYCLES`.
- Wave time shares (`SQ_*` / `SQ_WAVE_CYCLES`): issuing (`SQ_ACTIVE_INST_ANY`), blocked on issue
  (`SQ_WAIT_INST_ANY`), waiting in `s_waitcnt` or at a barrier (`SQ_WAIT_ANY`).
- HBM bytes: `FETCH_SIZE` and `WRITE_SIZE` (KiB) scaled by what the same counters read for a plain
  1 GiB device copy (`bench.py --only copy`), which reads FETCH_SIZE %d KiB and WRITE_SIZE %d KiB for
  1 048 576 KiB moved: FETCH_SIZE is multiplied by %.3f, WRITE_SIZE by %.3f.  Algorithmic bytes: each
  input read once and each output written once.
""" % (round(cf), round(cw), fs, ws))
    o.append("| Kernel | cycles per XCD | MFMA busy | LDS busy | co-exec | issuing / blocked / "
             "waiting | MFMA instr | VALU instr | transcendental share | LDS instr | bank conflicts "
             "| HBM read (MB) | alg. read (MB) | HBM write (MB) | alg. write (MB) |")
    o.append("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    order = sorted(raw, key=lambda k: ("pre" in k, "main" in k, "dq" in k, k))
    for k in order:
        d = raw[k]
        cyc = d["GRBM_GUI_ACTIVE"] / 8
        ar, aw = _alg_bytes(fam(k), w)
        mb = lambda x: "-" if x is None else "%.1f" % (x / 1e6)
        o.append("| `%s` | %d | %.1f%% | %.1f%% | %.1f%% | %d%% / %d%% / %d%% | %d | %d | %.1f%% "
                 "| %d | %d | %.1f | %s | %.1f | %s |" % (
                     short(k), round(cyc), 100 * d["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024),
                     100 * d["SQ_LDS_IDX_ACTIVE"] / (cyc * 256),
                     100 * d["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(1.0, d["SQ_VALU_MFMA_BUSY_CYCLES"]),
                     round(100 * d["SQ_ACTIVE_INST_ANY"] / d["SQ_WAVE_CYCLES"]),
                     round(100 * d["SQ_WAIT_INST_ANY"] / d["SQ_WAVE_CYCLES"]),
                     round(100 * d["SQ_WAIT_ANY"] / d["SQ_WAVE_CYCLES"]),
                     d["SQ_INSTS_MFMA"], d["SQ_INSTS_VALU"],
                     100 * d["SQ_INSTS_VALU_TRANS_F32"] / max(1.0, d["SQ_INSTS_VALU"]),
                     d["SQ_INSTS_LDS"], d["SQ_LDS_BANK_CONFLICT"],
                     d["FETCH_SIZE"] * 1024 * fs / 1e6, mb(ar), d["WRITE_SIZE"] * 1024 * ws / 1e6,
                     mb(aw)))
    if clk:
        o.append("\nMeasured clock.  Cycles per launch = `GRBM_GUI_ACTIVE` / 8 XCDs (wall cycles at "
                 "the shader clock), clock = cycles / the dispatch's duration (its start and end "
                 "timestamps), each the mean over the passes that hold the counter.  Fraction at "
                 "the clock = the kernel's credited algorithmic flops / (256 CUs x 4096 bf16 flops "
                 "per cycle, FP8 twice that, x cycles): its share of the dense peak at whatever "
                 "clock it runs at.  Fraction of the 2.4 GHz peak = the same flops over the mean "
                 "duration:\n")
        o.append("| Kernel | cycles per launch | clock (GHz) | mean duration (us) | fraction at the "
                 "clock | fraction of the 2.4 GHz peak |")
        o.append("|---|---|---|---|---|---|")
        for k in order:
            if k not in clk:
                continue
            cyc = sum(c * t for c, t in clk[k]) / len(clk[k])
            g = sum(c for c, _ in clk[k]) / len(clk[k])
            du = sum(t for _, t in clk[k]) / len(clk[k])
            per_cycle = PEAK_BF16_FLOP_PER_CYCLE * (2 if fam(k) == "attn_fwd_fp8_kernel" else 1)
            pk = PEAK_FP8_TFLOPS if fam(k) == "attn_fwd_fp8_kernel" else PEAK_BF16_TFLOPS
            fl = None
            if fam(k) in _CREDIT:
                kind, share = _CREDIT[fam(k)]
                if kind == "bwd":
                    fl = (share * 2.5 * fwd_flops(w.B, w.H, w.S, w.D, w.causal)
                          if w.backward else None)
                else:
                    fl = fwd_flops(w.B, w.H, w.S, w.D, w.causal)
            if fl is None:
                o.append("| `%s` | %d | %.3f | %.1f | - | - |" % (short(k), round(cyc), g, du / 1e3))
            else:
                o.append("| `%s` | %d | %.3f | %.1f | %.4f | %.4f |" % (
                    short(k), round(cyc), g, du / 1e3, fl / (per_cycle * cyc),
                    fl / (du * 1e-9) / 1e12 / pk))
    o.append("\nHBM bytes per launch (scaled): " + "; ".join(
        "`%s` read %d, write %d" % (fam(k), round(raw[k]["FETCH_SIZE"] * 1024 * fs),
                                    round(raw[k]["WRITE_SIZE"] * 1024 * ws)) for k in order) + "\n")
    o += ["Raw per-dispatch averages:\n", "| Kernel | Counter | Value |", "|---|---|---|"]
    for k in order:
        for c in sorted(raw[k]):
            v = raw[k][c]
            o.append("| `%s` | %s | %s |" % (short(k), c, ("%.1f" % v) if v != int(v) else "%d" % v))
    return "\n".join(o)


def lap_windows(path, steps, warmup):
    """The trace's durations over exactly the launches bench.py's live timing
    covers, for the two roofline kernels (a bench run traced with the same
    --steps and --warmup): the dK/dV kernel's steps-long instrumented step loop
    comes after its warmup launches, the timed steps and the median's steps; the causal
    S=8192 forward's leg laps after three warm-up launches and one warm launch.
    Returns markdown lines (trace mean and start-to-start mean per window)."""
    import csv
    import statistics
    import attn_inputs as ai
    n_rep = max(steps, 10)
    wb, wf = ai.WORKLOADS["bwd_causal_s4k"], ai.WORKLOADS["fwd_causal_s8k"]
    spans = {("attn_bwd_main_kernel", _grids(wb)["attn_bwd_main_kernel"]): (warmup + 2 * steps,
                                                                           steps, False),
             ("attn_fwd_kernel", _grids(wf)["attn_fwd_kernel"]): (4, n_rep, True)}
    runs = {k: [] for k in spans}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = r["Kernel_Name"]
            fam = name.split("<")[0].split("::")[-1].strip()
            targs = name.split("<")[1].split(">")[0].split(",") if "<" in name else []
            if len(targs) > 2 and targs[2].strip() == "true":
                continue   # the counting instantiation
            key = (fam, int(r["Grid_Size_X"]))
            if key in runs and targs[1].strip() == "true":
                runs[key].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out = []
    for (fam, grid), (first, n, back_to_back) in spans.items():
        t = sorted(runs[(fam, grid)])[first:first + n]
        if len(t) < 2:
            continue
        dur = [(e - b) / 1e3 for b, e in t]
        line = "- `%s` (grid %d), launches %d..%d in trace order: mean %.1f us, median %.1f us" % (
            fam, grid, first + 1, first + len(t), statistics.mean(dur), statistics.median(dur))
        if back_to_back:
            gap = [(t[i + 1][0] - t[i][0]) / 1e3 for i in range(len(t) - 1)]
            line += ", start-to-start %.1f us" % statistics.mean(gap)
        out.append(line)
    return out


SWEEP_TAUS = (0.0, 8.0, 16.0, 32.0, 64.0)
SWEEP_POLYS = (0, 8, 4)


def sweep_policy(args):
    """Time the long-sequence forward at every (rescale threshold, exponential
    policy) pair on each forward workload of at least 2048 keys (and the
    backward workload's forward), interleaving the pairs over three rounds so
    a drifting clock favours none; prints a markdown table of the median of
    the per-round means and one JSON line with the winner per workload."""
    import numpy as np
    import torch
    import attn_inputs as ai
    import exact_attention_128_amd as A
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    names = ("fwd_s2k", "bwd_causal_s4k", "fwd_causal_s8k", "fwd_stress_s16k")
    pairs = [(t, p) for p in SWEEP_POLYS for t in SWEEP_TAUS]
    result = {}
    lines = ["| Workload | tau | exp poly every | ms (median of 3 rounds x %d launches) | TFLOPS |"
             " vs library choice |" % args.steps, "|---|---|---|---|---|---|"]
    for name in names:
        w = ai.WORKLOADS[name]
        bits = ai.make_inputs(w.B, w.H, w.S, w.D, w.seed, stress=w.stress)
        q, k, v = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
        times = {pr: [] for pr in pairs}
        for _ in range(3):
            for (tau, poly) in pairs:
                run = lambda: A.fwd_out(q, k, v, o, lse, causal=w.causal, scale=w.scale,
                                        rescale_log2=tau, exp_poly_every=poly)
                for _ in range(args.warmup):
                    run()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(args.steps):
                    run()
                b.record(stream)
                torch.cuda.synchronize()
                times[(tau, poly)].append(a.elapsed_time(b) / args.steps)
        fl = fwd_flops(w.B, w.H, w.S, w.D, w.causal)
        med = {pr: float(np.median(t)) for pr, t in times.items()}
        lib_choice = A.default_policy(w.D, w.causal, w.S)
        best = min(med, key=med.get)
        result[name] = {"best": {"tau": best[0], "exp_poly_every": best[1], "ms": round(med[best], 4)},
                        "library_choice": {"tau": lib_choice[0], "exp_poly_every": lib_choice[1],
                                           "ms": round(med[lib_choice], 4)},
                        "ms": {"%g/%d" % pr: round(t, 4) for pr, t in med.items()}}
        for pr in pairs:
            lines.append("| %s | %g | %d | %.4f | %.1f | %+.1f%% |" % (
                name, pr[0], pr[1], med[pr], fl / (med[pr] * 1e-3) / 1e12,
                100.0 * (med[pr] / med[lib_choice] - 1.0)))
        log("sweep %s: best tau %g poly %d %.4f ms; library choice %s %.4f ms" % (
            name, best[0], best[1], med[best], lib_choice, med[lib_choice]))
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    print("\n".join(lines), flush=True)
    print(json.dumps({"sweep": result}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Under its power limit the GPU's clock settles over the first ~25 steps
    # of sustained load (the step time falls from ~760 to ~600 us on the
    # causal S=4096 workload) and then holds: 30 warm-up steps, then 100 timed
    # steps (~60 ms), so the timed window sees the sustained state.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="bwd_causal_s4k")
    ap.add_argument("--no-legs", action="store_true", help="skip the forward-only legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time for the oracle sample of the step's workload")
    ap.add_argument("--cpu-leg-seconds", type=float, default=2.0,
                    help="target CPU time for the oracle sample of each forward leg")
    ap.add_argument("--only", default=None,
                    help="profiling driver: run one workload's kernels --steps times after "
                         "--warmup runs and exit (a workload name, 'copy' for a plain "
                         "1 GiB device copy that calibrates the HBM byte counters, or 'gemm' "
                         "for the bf16 8192^3 library GEMM that calibrates the MFMA clock)")
    ap.add_argument("--trace-summary", default=None, metavar="KERNEL_TRACE_CSV",
                    help="print a per-workload markdown summary of a rocprofv3 kernel-trace "
                         "CSV and exit (no GPU needed)")
    ap.add_argument("--pmc-summary", nargs=2, default=None, metavar=("PMC_DIR", "WORKLOAD"),
                    help="print the markdown summary of one workload's counter passes "
                         "(rocprofv3 --pmc CSVs under PMC_DIR) and exit (no GPU needed)")
    ap.add_argument("--sweep-policy", action="store_true",
                    help="time the forward at every (rescale threshold, exponential policy) "
                         "pair on the forward workloads and print the table (uses --steps, "
                         "--warmup per pair and round)")
    args = ap.parse_args()
    if args.sweep_policy:
        sweep_policy(args)
        return
    if args.trace_summary is not None:
        print(trace_summary(args.trace_summary))
        print("\nThe launches the live laps time (this run's --steps %d --warmup %d):\n" % (
            args.steps, args.warmup))
        print("\n".join(lap_windows(args.trace_summary, args.steps, args.warmup)))
        return
    if args.pmc_summary is not None:
        print(pmc_summary(*args.pmc_summary))
        return
    if args.only is not None:
        run_only(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library's path has no multi-GPU "
              "step (independent heads shard with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import attn_inputs as ai
    import exact_attention_128_amd as A

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = ai.WORKLOADS[args.workload]
    B, H, S, D, causal, scale = w.B, w.H, w.S, w.D, w.causal, w.scale
    log("workload", w.name, w.describe())

    bits = ai.make_inputs(B, H, S, D, w.seed, stress=w.stress, with_dout=True)
    q, k, v, do = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(A.bwd_workspace_size(B, H, S, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        A.fwd_out(q, k, v, o, lse, causal=causal, scale=scale)
        A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal, scale=scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed region: K steps between two events (an event marker between
    # steps would add a few microseconds of idle GPU to each).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / args.steps
    # the per-step median from the same K steps run once more with an event
    # after each
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    sev[0].record(stream)
    for i in range(args.steps):
        step()
        sev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_step_median = float(np.median([sev[i].elapsed_time(sev[i + 1])
                                      for i in range(args.steps)]))
    f_fwd = fwd_flops(B, H, S, D, causal)
    f_bwd = 2.5 * f_fwd
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    log("step: %.3f ms  %.1f TFLOPS (wall %.3f ms/step)" % (ms_step, value,
                                                          1e3 * t_wall / args.steps))

    # The same K steps once more with an event between the step's kernels
    # (forward | dQ and row statistics | dK/dV, the backward split into its two
    # launches, the same GPU work): each kernel's duration in the step, where
    # it shares the clock with the other two.  Each event marker costs a few
    # microseconds of idle time, which is why the step itself is timed above
    # without them.
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps + 1)]
    kev[0].record(stream)
    for i in range(args.steps):
        A.fwd_out(q, k, v, o, lse, causal=causal, scale=scale)
        kev[3 * i + 1].record(stream)
        A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal, scale=scale,
                  phases=A.BWD_DQ)
        kev[3 * i + 2].record(stream)
        A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal, scale=scale,
                  phases=A.BWD_MAIN)
        kev[3 * i + 3].record(stream)
    torch.cuda.synchronize()
    in_step = {n: [kev[3 * i + j].elapsed_time(kev[3 * i + j + 1]) for i in range(args.steps)]
               for j, n in enumerate(("fwd", "dq", "main"))}
    ms_main = float(np.mean(in_step["main"]))
    med_main = float(np.median(in_step["main"]))
    ms_dq = float(np.mean(in_step["dq"]))
    med_dq = float(np.median(in_step["dq"]))
    ms_fwd_step = float(np.mean(in_step["fwd"]))

    def time_launches(fn, n):
        """Mean launch time in ms over n back-to-back launches between two HIP
        events on the launch stream (an event after each launch would add its
        marker's few microseconds to every launch); the per-launch times of n
        more launches, an event after each, go to `laps` for the median."""
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record(stream)
        for i in range(n):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        laps.append([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
        return a.elapsed_time(b) / n

    laps = []

    def last_median():
        return float(np.median(laps[-1]))

    # The dominant kernel is the backward's dK/dV kernel (run PRE once so the
    # workspace holds the row statistics).  Its algorithmic work is four of the
    # backward's five products (S, dP, dV, dK): 0.8 of the backward FLOPs.  The
    # dQ kernel's algorithmic work is the fifth (dQ); it also recomputes S and
    # dP, which the count leaves out.
    # Also each kernel alone, back to back (context: a lone run of the heaviest
    # kernel holds the clock lower than the mixed step does).
    A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal, scale=scale, phases=A.BWD_PRE)
    n_rep = max(args.steps, 10)
    ms_main_alone = time_launches(lambda: A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws,
                                                    causal=causal, scale=scale,
                                                    phases=A.BWD_MAIN), n_rep)
    ms_dq_alone = time_launches(lambda: A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws,
                                                  causal=causal, scale=scale, phases=A.BWD_DQ),
                                n_rep)
    ms_fwd = time_launches(lambda: A.fwd_out(q, k, v, o, lse, causal=causal, scale=scale), n_rep)
    med_fwd = last_median()
    ms_bwd = time_launches(lambda: A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal,
                                             scale=scale), n_rep)
    med_bwd = last_median()
    main_tflops = 0.8 * f_bwd / (ms_main * 1e-3) / 1e12
    dq_alg_tflops = 0.2 * f_bwd / (ms_dq * 1e-3) / 1e12
    dq_exec_tflops = 0.6 * f_bwd / (ms_dq * 1e-3) / 1e12
    log("in the step: dK/dV %.3f ms (%.1f TFLOPS), dQ %.3f ms (%.1f executed TFLOPS), fwd %.3f ms"
        % (ms_main, main_tflops, ms_dq, dq_exec_tflops, ms_fwd_step))
    log("alone: dK/dV %.3f ms, dQ %.3f ms, fwd %.3f ms, bwd total %.3f ms" % (
        ms_main_alone, ms_dq_alone, ms_fwd, ms_bwd))

    legs = {}
    cpu_legs = {}
    fwd_roof = None
    short_roof = None
    gemm_tflops = None
    if not args.no_cpu_baseline:
        import oracle
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        cores = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
        oracle.set_threads(cores)
    if not args.no_legs:
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
        for name in ("tiny", "fwd_s2k", "fwd_causal_s8k", "fwd_stress_s16k",
                     *ai.SHORT_WORKLOADS):
            lw = ai.ALL_WORKLOADS[name]
            lb = ai.workload_inputs(lw)
            lq, lk, lv = (ai.to_torch_bf16(lb[n], dev) for n in ("q", "k", "v"))
            lo = torch.empty_like(lq)
            ll = torch.empty((lw.B, lw.H, lw.S), dtype=torch.float32, device=dev)
            for _ in range(3):
                A.fwd_out(lq, lk, lv, lo, ll, causal=lw.causal, scale=lw.scale)
            ms = time_launches(lambda: A.fwd_out(lq, lk, lv, lo, ll, causal=lw.causal,
                                                 scale=lw.scale), n_rep)
            med = last_median()
            fl = fwd_flops(lw.B, lw.H, lw.S, lw.D, lw.causal)
            tf = fl / (ms * 1e-3) / 1e12
            # algorithmic HBM bytes: Q, K, V read and O written (bf16), LSE (fp32)
            nbytes = 8.0 * lw.B * lw.H * lw.S * lw.D + 4.0 * lw.B * lw.H * lw.S
            gbs = nbytes / (ms * 1e-3) / 1e9
            legs[name] = {"shape": [lw.B, lw.H, lw.S, lw.D], "causal": lw.causal,
                          "ms": round(ms, 4), "median_ms": round(med, 4), "tflops": round(tf, 2),
                          "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                          "frac_peak_median": round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
            log("fwd leg %s: %.4f ms  %.1f TFLOPS (%.1f%%)  %.1f GB/s algorithmic HBM" % (
                name, ms, tf, 100 * tf / PEAK_BF16_TFLOPS, gbs))
            if not args.no_cpu_baseline:
                cpu_legs[name] = oracle_fwd_sample(lw, lb, args.cpu_leg_seconds)
                log("  cpu oracle %s: %s" % (name, cpu_legs[name]))
            if lw.causal and lw.S > 128:
                # untimed: how often the conditional rescale fires (the counting
                # forward, attn_fwd_rescale_events), at the library's threshold
                # 2^64, at 2^32 and at FA4's 2^8
                ev = {}
                for tau in (64.0, 32.0, 8.0):
                    _, _, tests, fired = A.fwd_rescale_events(lq, lk, lv, causal=lw.causal,
                                                              scale=lw.scale, rescale_log2=tau)
                    ev["tau%d" % tau] = {"tests": tests, "fired": fired,
                                         "rate": round(fired / max(1, tests), 4)}
                legs[name]["rescale_events"] = ev
                log("  rescale events %s: %s" % (name, ev))
            del lq, lk, lv, lo, ll
            torch.cuda.empty_cache()
        # The FP8 (E4M3) forward on the causal S=8192 shape (the same draws as
        # the bf16 leg, quantized per tensor), against the FP8 dense peak.
        fw = ai.FP8_WORKLOAD
        b8 = ai.make_inputs_fp8(fw.B, fw.H, fw.S, fw.D, fw.seed)
        q8, k8, v8 = (ai.to_torch_u8(b8[n], dev) for n in ("q", "k", "v"))
        o8 = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
        l8 = torch.empty((fw.B, fw.H, fw.S), dtype=torch.float32, device=dev)
        run8 = lambda: A.fwd_fp8_out(q8, k8, v8, b8["q_descale"], b8["k_descale"],
                                     b8["v_descale"], o8, l8, causal=fw.causal, scale=fw.scale)
        for _ in range(3):
            run8()
        ms = time_launches(run8, n_rep)
        med = last_median()
        fl = fwd_flops(fw.B, fw.H, fw.S, fw.D, fw.causal)
        tf = fl / (ms * 1e-3) / 1e12
        legs[fw.name] = {"shape": [fw.B, fw.H, fw.S, fw.D], "causal": fw.causal, "dtype": "e4m3",
                         "ms": round(ms, 4), "median_ms": round(med, 4), "tflops": round(tf, 2),
                         "frac_peak_fp8": round(tf / PEAK_FP8_TFLOPS, 4),
                         "frac_peak_bf16": round(tf / PEAK_BF16_TFLOPS, 4),
                         "speedup_vs_bf16": round(legs["fwd_causal_s8k"]["ms"] / ms, 3)}
        log("fwd leg %s: %.4f ms  %.1f TFLOPS (%.1f%% of the FP8 peak, %.2fx the bf16 leg)" % (
            fw.name, ms, tf, 100 * tf / PEAK_FP8_TFLOPS, legs[fw.name]["speedup_vs_bf16"]))
        del q8, k8, v8, o8, l8
        torch.cuda.empty_cache()
        # Context for the MFMA peak on this part: a plain vendor-library bf16 GEMM
        # (hipBLASLt through torch.matmul, contiguous 8192^3 operands, fp32
        # accumulate) timed the same way.  Not part of the attention path.
        n = 8192
        ga = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        gb = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        gc = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(ga, gb, out=gc)
        ms = time_launches(lambda: torch.matmul(ga, gb, out=gc), n_rep)
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        gemm_tflops = tf
        legs["library_gemm"] = {"op": "torch.matmul bf16 8192x8192x8192 (hipBLASLt)",
                                "ms": round(ms, 4), "median_ms": round(last_median(), 4),
                                "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        log("library GEMM (hipBLASLt bf16 8192^3): %.4f ms  %.1f TFLOPS (%.1f%%)" % (
            ms, tf, 100 * tf / PEAK_BF16_TFLOPS))
        del ga, gb, gc
        torch.cuda.empty_cache()
        # Context for the HBM peak: a plain 1 GiB device-to-device copy (torch's
        # copy kernel; 2 GiB moved per launch) timed the same way.  Not part of
        # the attention path.
        nb = 1 << 30
        csrc = torch.ones(nb, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        for _ in range(3):
            cdst.copy_(csrc)
        ms = time_launches(lambda: cdst.copy_(csrc), n_rep)
        copy_gbs = 2.0 * nb / (ms * 1e-3) / 1e9
        legs["device_copy"] = {"op": "torch copy_ of 1 GiB (read + write)", "ms": round(ms, 4),
                               "median_ms": round(last_median(), 4), "hbm_gbs": round(copy_gbs, 1),
                               "hbm_frac": round(copy_gbs / PEAK_HBM_GBS, 4)}
        log("device copy (1 GiB): %.4f ms  %.1f GB/s (%.1f%% of %.0f)" % (
            ms, copy_gbs, 100 * copy_gbs / PEAK_HBM_GBS, PEAK_HBM_GBS))
        del csrc, cdst
        torch.cuda.empty_cache()
        for name in ai.SHORT_WORKLOADS:
            legs[name]["hbm_frac_vs_device_copy"] = round(legs[name]["hbm_gbs"] / copy_gbs, 4)
        sh = legs["fwd_short_s128_h4096"]
        short_roof = {"kernel": "attn_fwd_short_kernel<128,non-causal>",
                      "workload": "fwd_short_s128_h4096", "bound": "hbm",
                      "achieved": sh["hbm_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": sh["hbm_frac"], "ms": sh["ms"], "median_ms": sh["median_ms"],
                      "frac_vs_device_copy": sh["hbm_frac_vs_device_copy"]}
        c3 = legs["fwd_causal_s8k"]
        fwd_roof = {"kernel": "attn_fwd_kernel<128,causal>", "workload": "fwd_causal_s8k",
                    "bound": "mfma", "achieved": c3["tflops"], "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": c3["frac_peak"], "ms": c3["ms"],
                    "median_ms": c3["median_ms"], "frac_median": c3["frac_peak_median"],
                    "frac_vs_library_gemm": round(c3["tflops"] / gemm_tflops, 4),
                    "traffic": measured_traffic("fwd_causal_s8k", FWD_TRAFFIC, FWD_TRAFFIC_SOURCES)}
        cw = ai.WORKLOADS["fwd_causal_s8k"]
        fwd_roof.update(at_clock(fwd_flops(cw.B, cw.H, cw.S, cw.D, cw.causal), c3["ms"],
                                 "fwd_causal_s8k", FWD_TRAFFIC, FWD_TRAFFIC_SOURCES))

    cpu = None
    if not args.no_cpu_baseline:
        qs, ks, vs, dos = (bits[n].reshape(B * H, S, D) for n in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        heads = 0
        while heads < B * H and time.perf_counter() - t0 < args.cpu_seconds:
            oracle.attn_bwd_head(*(ai.bf16_bits_to_f64(x[heads]) for x in (qs, ks, vs, dos)),
                                 scale, causal)
            heads += 1
        dt = time.perf_counter() - t0
        per_head = (f_fwd + f_bwd) / (B * H)
        cpu = {"value": round(heads * per_head / dt / 1e12, 6), "unit": "TFLOPS",
               "cores": oracle.max_threads(), "kind": "oracle",
               "sample": "%d of %d heads of the workload, fp64 forward+backward per head, "
                         "%.1f s" % (heads, B * H, dt),
               "per_config": cpu_legs}
        log("cpu oracle: %s" % cpu)

    main_clk = at_clock(0.8 * f_bwd, ms_main, w.name)
    out = {
        "metric": "attention fwd/bwd TFLOPS (bf16, D=128) and % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 inputs, seed %d)" % w.seed,
        "config": {"workload": w.name, "B": B, "H": H, "S": S, "D": D, "causal": causal,
                   "step": "forward + backward", "frac_peak": round(value / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"kernel": "attn_bwd_main_kernel<128,causal>", "bound": "mfma",
                     "achieved": round(main_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(main_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name), "ms": round(ms_main, 4),
                     "median_ms": round(med_main, 4),
                     "frac_median": round(0.8 * f_bwd / (med_main * 1e-3) / 1e12 /
                                          PEAK_BF16_TFLOPS, 4),
                     "frac_vs_library_gemm": (round(main_tflops / gemm_tflops, 4)
                                              if gemm_tflops else None),
                     "timed": "in the step, %d steps" % args.steps,
                     "alone_ms": round(ms_main_alone, 4),
                     **main_clk},
        "dq_kernel": {"kernel": "attn_bwd_dq_kernel<128,causal>", "ms": round(ms_dq, 4),
                      "median_ms": round(med_dq, 4), "alone_ms": round(ms_dq_alone, 4),
                      "algorithmic_tflops": round(dq_alg_tflops, 1),
                      "executed_tflops": round(dq_exec_tflops, 1),
                      "executed_frac": round(dq_exec_tflops / PEAK_BF16_TFLOPS, 4)},
        "ms_per_step_median": round(ms_step_median, 4),
        "step_at_clock": at_clock(f_fwd + f_bwd, ms_step, w.name, STEP_CYCLES, STEP_SOURCES),
        "fwd_ms": round(ms_fwd, 4),
        "fwd_median_ms": round(med_fwd, 4),
        "bwd_ms": round(ms_bwd, 4),
        "bwd_median_ms": round(med_bwd, 4),
        "fwd_tflops": round(f_fwd / (ms_fwd * 1e-3) / 1e12, 1),
        "bwd_tflops": round(f_bwd / (ms_bwd * 1e-3) / 1e12, 1),
        "fwd_roofline": fwd_roof,
        "short_roofline": short_roof,
        "legs": legs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def run_only(args):
    """Run a single workload (or the calibration copy) for a profiler; prints
    one line naming what ran."""
    import torch
    import attn_inputs as ai
    import exact_attention_128_amd as A

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.only == "gemm":
        n = 8192
        ga = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        gb = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        gc = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        for _ in range(args.warmup + args.steps):
            torch.matmul(ga, gb, out=gc)
        torch.cuda.synchronize()
        print("ran gemm: %d launches of a bf16 %d^3 library GEMM" % (args.warmup + args.steps, n),
              flush=True)
        return
    if args.only == "copy":
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("ran copy: %d launches of a %d-byte device copy" % (args.warmup + args.steps, n),
              flush=True)
        return
    if args.only == ai.FP8_WORKLOAD.name:
        w = ai.FP8_WORKLOAD
        b8 = ai.make_inputs_fp8(w.B, w.H, w.S, w.D, w.seed)
        q8, k8, v8 = (ai.to_torch_u8(b8[n], dev) for n in ("q", "k", "v"))
        o8 = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
        l8 = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
        for _ in range(args.warmup + args.steps):
            A.fwd_fp8_out(q8, k8, v8, b8["q_descale"], b8["k_descale"], b8["v_descale"], o8, l8,
                          causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        print("ran %s: %d launches (FP8 forward)" % (w.name, args.warmup + args.steps), flush=True)
        return
    w = ai.ALL_WORKLOADS[args.only]
    bits = ai.make_inputs(w.B, w.H, w.S, w.D, w.seed, stress=w.stress, with_dout=w.backward)
    q, k, v = (ai.to_torch_bf16(bits[n], dev) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    if not w.backward:
        for _ in range(args.warmup + args.steps):
            A.fwd_out(q, k, v, o, lse, causal=w.causal, scale=w.scale)
    else:
        do = ai.to_torch_bf16(bits["do"], dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(A.bwd_workspace_size(w.B, w.H, w.S, w.D), dtype=torch.uint8, device=dev)
        A.fwd_out(q, k, v, o, lse, causal=w.causal, scale=w.scale)
        for _ in range(args.warmup + args.steps):
            A.bwd_out(q, k, v, o, lse, do, dq, dk, dv, ws, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    print("ran %s: %d launches (%s)" % (w.name, args.warmup + args.steps,
                                       "backward after one forward" if w.backward else "forward"),
          flush=True)


if __name__ == "__main__":
    main()
