"""Ahead-of-time build of libattn.so for gfx950 with hipcc.

Each HIP translation unit under csrc/ is compiled to an object file (in
parallel), then linked into exact_attention_128_amd/libattn.so.  The build
always recompiles; the library is loaded from this directory.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libattn.so")
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


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, outdir: str, extra) -> str:
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + PER_SOURCE.get(os.path.basename(src), []) + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(extra=(), out: str = LIB, verbose: bool = False) -> str:
    outdir = os.path.join(ROOT, "_build")
    os.makedirs(outdir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, outdir, extra), srcs))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
