"""Ahead-of-time build of libattn.so for gfx950 with hipcc.

Each HIP translation unit under csrc/ is compiled to an object file (in
parallel), then linked into exact_attention_128_amd/libattn.so.  The build
always recompiles; the library is loaded from this directory.
"""
from __future__ import annotations

import concurrent.futures
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libattn.so")
# The LDS race-check build: the same sources and C ABI with every direct-to-LDS
# load preceded by a NaN pattern over its destination (gfx950.h, lds_dma16).
# Debug only; nothing on the product path loads it.
LIB_LDS_POISON = os.path.join(HERE, "libattn_lds_poison.so")
POISON_FLAGS = ["-DATTN_LDS_POISON=1"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-std=c++20", "-O3", "-fPIC", "--offload-arch=" + ARCH,
    # no packed-fp32 VALU forms: keep every fp32 op scalar per lane
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


# Per-source flags.  attn_bwd.hip: one wave per SIMD may use 512 registers,
# and with that budget the compiler would give every matrix product an AGPR
# accumulator, so the softmax would copy each score back to a VGPR first;
# the VGPR form keeps the scores in VGPRs (the dK/dV accumulators still spill
# to AGPRs where needed).
PER_SOURCE = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


# Every compile asks the compiler for its per-kernel resource report (VGPRs,
# AGPRs, scratch bytes per lane, spills, occupancy, LDS); the build refuses a
# kernel that uses scratch memory or spills vector registers, since a spill in
# these kernels costs far more than it saves (one measured case: +21 % forward
# time).  The report goes to _build/kernel_resources.json.
RESOURCE_FLAG = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(.*?):\s+(\S+) \[-Rpass-analysis=kernel-resource-usage\]")
_NAME = re.compile(r"remark: Function Name: (\S+) \[-Rpass-analysis")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def parse_resource_remarks(text: str) -> dict:
    """{mangled kernel name: {field: value}} from the compiler's resource remarks."""
    kernels, cur = {}, None
    for line in text.splitlines():
        m = _NAME.search(line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = _REMARK.search(line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return kernels


def resource_violations(kernels: dict) -> list:
    """Kernels that use scratch memory, spill vector registers or need a dynamic
    stack.  (Scalar registers spilled into vector-register lanes touch no memory
    and are only reported.)"""
    bad = []
    for name, r in kernels.items():
        if (int(r.get("ScratchSize [bytes/lane]", "0")) != 0 or int(r.get("VGPRs Spill", "0")) != 0
                or r.get("Dynamic Stack", "False") != "False"):
            bad.append((name, r))
    return bad


def _quiet(text: str) -> str:
    """Compiler output minus the resource remarks (and their source excerpts)
    and the host pass's note about the GPU-only feature flag."""
    keep = []
    for l in text.splitlines():
        if "packed-fp32-ops' is not a recognized feature" in l or RESOURCE_FLAG in l:
            continue
        if re.match(r"^\s*\d*\s*\|", l):
            continue
        keep.append(l)
    return "\n".join(keep)


def compile_source(src: str, obj: str, extra=()) -> dict:
    """Compile one HIP source to obj; returns its kernels' resource report."""
    cmd = ([HIPCC] + COMMON + PER_SOURCE.get(os.path.basename(src), []) + [RESOURCE_FLAG] +
           list(extra) + ["-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = _quiet(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if msg.strip():
        print(msg, file=sys.stderr)
    return parse_resource_remarks(r.stdout + r.stderr)


def _compile(src: str, outdir: str, extra):
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    return obj, compile_source(src, obj, extra)


def build(extra=(), out: str = LIB, verbose: bool = False, objdir: str = "_build",
          guard: bool = True) -> str:
    """Compile every source and link out.  guard: refuse kernels that use
    scratch memory or spill vector registers (the product library); the
    race-check build only reports them, since its extra stores and waits may
    spill where the product kernels fit, which costs it speed, not
    correctness."""
    outdir = os.path.join(ROOT, objdir)
    os.makedirs(outdir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = list(ex.map(lambda s: _compile(s, outdir, extra), srcs))
    objs = [o for o, _ in done]
    report = {}
    for _, k in done:
        report.update(k)
    with open(os.path.join(outdir, "kernel_resources.json"), "w") as fh:
        json.dump(report, fh, indent=1, sort_keys=True)
    bad = resource_violations(report)
    if bad and not guard:
        print("note (%s): %d kernel(s) use scratch memory:\n%s" % (
            os.path.basename(out), len(bad), "\n".join("  %s" % b[0] for b in bad)),
            file=sys.stderr)
    elif bad:
        raise RuntimeError("kernels using scratch memory or spilling registers:\n" +
                           "\n".join("  %s: %s" % b for b in bad))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def build_all(verbose: bool = False) -> None:
    """The product library and the LDS race-check build."""
    build(verbose=verbose)
    build(extra=POISON_FLAGS, out=LIB_LDS_POISON, verbose=verbose,
          objdir=os.path.join("_build", "lds_poison"), guard=False)


if __name__ == "__main__":
    build_all(verbose=True)
