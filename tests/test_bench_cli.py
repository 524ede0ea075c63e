"""CPU checks of bench.py: a request for more than one GPU is refused with a
message (the path has no multi-GPU step), the JSON-producing entry parses its
flags, the recorded HBM traffic is dropped once its kernel sources change, and
the kernel-trace and hardware-counter summaries compute what they state."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_help_lists_the_contract_flags():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--only"):
        assert flag in r.stdout


def _bench():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_record_is_dropped_once_its_sources_change(tmp_path):
    """measured_traffic reports the recorded bytes only for the workload it was
    taken on and only while the digest of the named sources matches."""
    import hashlib
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel v1")
    rel = os.path.relpath(str(src), ROOT)
    rec = {"workload": "w", "read_bytes": 10, "write_bytes": 5,
           "sources_sha256": hashlib.sha256(b"kernel v1").hexdigest()}
    assert b.measured_traffic("w", rec, (rel,)) == 15
    assert b.measured_traffic("other", rec, (rel,)) is None
    src.write_bytes(b"kernel v2")
    assert b.measured_traffic("w", rec, (rel,)) is None


def _write_trace(path, rows):
    import csv
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Grid_Size_X", "Start_Timestamp",
                                             "End_Timestamp"])
        wr.writeheader()
        for name, grid, dur_ns in rows:
            wr.writerow({"Kernel_Name": name, "Grid_Size_X": grid, "Start_Timestamp": 1000,
                         "End_Timestamp": 1000 + dur_ns})


def test_trace_summary_names_workloads_and_rates(tmp_path):
    """A kernel-trace CSV is grouped by (kernel, grid); the grid names the
    workload and the rate is the workload's algorithmic flops over the mean."""
    import attn_inputs as ai
    b = _bench()
    w = ai.WORKLOADS["fwd_causal_s8k"]
    grid = w.B * w.H * (w.S // 256) * 512
    f8 = ai.FP8_WORKLOAD
    p = tmp_path / "trace.csv"
    _write_trace(p, [("void attn::attn_fwd_kernel<128, true, false, 0>(attn::FwdParams)", grid,
                      1_000_000)] * 3 +
                 [("void attn::attn_fwd_fp8_kernel<128, true>(attn::Fp8FwdParams)", grid, 500_000)])
    md = b.trace_summary(str(p))
    lines = [l for l in md.splitlines() if "attn_fwd" in l]
    assert len(lines) == 2
    fwd = next(l for l in lines if "attn_fwd_kernel" in l)
    tf = b.fwd_flops(w.B, w.H, w.S, w.D, True) / 1e-3 / 1e12
    cells = [c.strip() for c in fwd.split("|")]
    assert "fwd_causal_s8k" in cells and "3" in cells
    assert ("%.1f" % tf) in cells
    fp8 = next(l for l in lines if "attn_fwd_fp8_kernel" in l)
    tf8 = b.fwd_flops(f8.B, f8.H, f8.S, f8.D, True) / 0.5e-3 / 1e12
    assert f8.name in fp8 and ("%.1f" % tf8) in fp8
    assert ("%.4f of %.1f" % (tf8 / b.PEAK_FP8_TFLOPS, b.PEAK_FP8_TFLOPS)) in fp8


def test_pmc_summary_scales_bytes_by_the_copy(tmp_path):
    """The HBM byte counters are scaled by what they read for the 1 GiB copy,
    and the derived shares follow the stated formulas."""
    import csv
    b = _bench()
    name = "void attn::attn_fwd_kernel<128, true, false, 0>(attn::FwdParams)"

    def put(n, wl, kernel, values):
        d = tmp_path / ("p%d_%s" % (n, wl))
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as fh:
            wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            wr.writeheader()
            for c, v in values.items():
                wr.writerow({"Kernel_Name": kernel, "Counter_Name": c, "Counter_Value": v})

    put(3, "copy", "__amd_rocclr_copyBuffer", {"FETCH_SIZE": 524288})
    put(4, "copy", "__amd_rocclr_copyBuffer", {"WRITE_SIZE": 1048576})
    cyc = 8000
    vals = {1: {"SQ_WAVE_CYCLES": 1000, "SQ_BUSY_CYCLES": 1, "SQ_VALU_MFMA_BUSY_CYCLES": 512000,
                "SQ_INSTS_MFMA": 7, "SQ_INSTS_LDS": 3, "SQ_LDS_BANK_CONFLICT": 0,
                "SQ_WAIT_INST_LDS": 0, "GRBM_GUI_ACTIVE": cyc},
            2: {"SQ_INSTS_VALU": 100, "SQ_INSTS_VALU_TRANS_F32": 25, "SQ_ACTIVE_INST_VALU": 1,
                "SQ_ACTIVE_INST_ANY": 400, "SQ_WAIT_ANY": 300, "SQ_WAIT_INST_ANY": 200,
                "SQ_INSTS_SALU": 1, "GRBM_GUI_ACTIVE": cyc},
            3: {"FETCH_SIZE": 1000},
            4: {"WRITE_SIZE": 3000},
            5: {"SQ_LDS_IDX_ACTIVE": 64000, "SQ_LDS_CMD_FIFO_FULL": 0,
                "SQ_VALU_MFMA_COEXEC_CYCLES": 256000, "SQ_ACTIVE_INST_LDS": 1,
                "SQ_ACTIVE_INST_SCA": 1, "SQ_ACTIVE_INST_VMEM": 1, "SQ_ACTIVE_INST_MISC": 1,
                "GRBM_GUI_ACTIVE": cyc}}
    for n, v in vals.items():
        put(n, "fwd_causal_s8k", name, v)
    md = b.pmc_summary(str(tmp_path), "fwd_causal_s8k")
    row = next(l for l in md.splitlines() if l.startswith("| `attn::attn_fwd_kernel"))
    cells = [c.strip() for c in row.split("|")[1:-1]]
    # cycles per XCD, MFMA busy (512000 / (1000 x 1024)), LDS busy (64000 / (1000 x 256)),
    # co-exec, issuing / blocked / waiting, transcendental share
    assert cells[1:6] == ["1000", "50.0%", "25.0%", "50.0%", "40% / 20% / 30%"]
    assert cells[8] == "25.0%"
    # FETCH_SIZE x 2 (the copy's fetch reads half the bytes moved), WRITE_SIZE x 1
    assert cells[11] == "%.1f" % (1000 * 1024 * 2 / 1e6)
    assert cells[13] == "%.1f" % (3000 * 1024 / 1e6)
    assert "read %d, write %d" % (1000 * 1024 * 2, 3000 * 1024) in md


def test_cycle_record_gives_the_fraction_at_the_clock(tmp_path):
    """at_clock: flops over (peak flops per cycle x profiled cycles), the live
    clock as cycles over the live duration, and nothing once the sources
    change."""
    import hashlib
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_bytes(b"v1")
    rel = os.path.relpath(str(src), ROOT)
    rec = {"workload": "w", "read_bytes": 1, "write_bytes": 1, "cycles": 1_000_000,
           "sources_sha256": hashlib.sha256(b"v1").hexdigest()}
    flops = 0.5 * 256 * 4096 * 1_000_000
    r = b.at_clock(flops, 0.625, "w", rec, (rel,))
    assert r == {"cycles_profiled": 1_000_000, "frac_at_clock": 0.5, "clock_ghz_live": 1.6}
    src.write_bytes(b"v2")
    assert b.at_clock(flops, 0.625, "w", rec, (rel,))["frac_at_clock"] is None
