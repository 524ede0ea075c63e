"""CPU checks of the build's register guard: every production kernel compiles
with no scratch memory and no spilled vector registers, and the guard does
catch a kernel that spills (a probe kernel with a dynamically indexed local
array, which the compiler must place in scratch memory)."""
import concurrent.futures
import os

import pytest

from exact_attention_128_amd import build as B

SPILLING_KERNEL = r"""
#include <hip/hip_runtime.h>
__global__ void spill_probe(const float* in, float* out, int n) {
  float a[96];
  for (int i = 0; i < 96; ++i) a[i] = in[(threadIdx.x + i) % n];
  out[threadIdx.x] = a[(threadIdx.x * 7 + n) % 96];
}
"""

# kernel families every build must contain (mangled-name prefixes)
EXPECTED = ("_ZN4attn15attn_fwd_kernel", "_ZN4attn18attn_bwd_dq_kernel",
            "_ZN4attn20attn_bwd_main_kernel", "_ZN4attn19attn_bwd_pre_kernel")


def test_production_kernels_use_no_scratch(tmp_path):
    srcs = B.sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        reports = list(ex.map(lambda s: B.compile_source(s, str(tmp_path / (os.path.basename(s) +
                                                                             ".o"))), srcs))
    kernels = {}
    for r in reports:
        kernels.update(r)
    for prefix in EXPECTED:
        assert any(k.startswith(prefix) for k in kernels), "no %s* in the report" % prefix
    for name, r in kernels.items():
        print(name, "VGPRs", r["VGPRs"], "AGPRs", r["AGPRs"], "scratch",
              r["ScratchSize [bytes/lane]"], "occupancy", r["Occupancy [waves/SIMD]"])
    assert B.resource_violations(kernels) == []


def test_guard_catches_a_spill(tmp_path):
    src = tmp_path / "spill_probe.hip"
    src.write_text(SPILLING_KERNEL)
    kernels = B.compile_source(str(src), str(tmp_path / "spill_probe.o"))
    assert list(kernels) == ["_Z11spill_probePKfPfi"]
    r = kernels["_Z11spill_probePKfPfi"]
    assert int(r["ScratchSize [bytes/lane]"]) > 0
    bad = B.resource_violations(kernels)
    assert [name for name, _ in bad] == ["_Z11spill_probePKfPfi"]
