"""Host-side sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer,
no recovery), run on the CPU:

* the fp64 oracle (oracle.c, gcc): every entry point on small random inputs,
  the edge cases (S = 1, one head, the whole causal tail) and invalid
  arguments;
* the C ABI's host layer (attn_api.hip, attn_noalloc.hip; sanitizers on the
  host pass only, the device pass untouched) linked against stub launchers
  that record the launch instead of starting a kernel: every validation path
  of every entry point, extreme shapes (int-range dimensions whose products
  overflow 32 and 40 bits), and the valid paths down to the launch.

A sanitizer finding aborts the driver, which fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="-1",
           ROCR_VISIBLE_DEVICES="-1", OMP_NUM_THREADS="2")

ORACLE_DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
int oracle_attn_fwd(const double*, const double*, const double*, long, long, long, long, double, int, double*, double*);
int oracle_attn_fwd_rows(const double*, const long*, long, const double*, const double*, long, long, double, int, double*, double*);
int oracle_attn_bwd_head(const double*, const double*, const double*, const double*, long, long, double, int, double*, double*, double*, double*, double*);
int oracle_attn_bwd(const double*, const double*, const double*, const double*, long, long, long, long, double, int, double*, double*, double*);
int oracle_attn_bwd_causal_tail(const double*, const double*, long, const double*, const double*, long, long, double, double*, double*, double*);
static double* rnd(long n) {
  double* p = (double*)malloc(sizeof(double) * (size_t)n);
  for (long i = 0; i < n; ++i) p[i] = (double)((i * 7919 + 13) % 1000) / 250.0 - 2.0;
  return p;
}
int main(void) {
  const long shapes[][4] = {{1, 1, 1, 4}, {2, 3, 17, 8}, {1, 2, 40, 16}};
  for (int t = 0; t < 3; ++t) {
    const long B = shapes[t][0], H = shapes[t][1], S = shapes[t][2], D = shapes[t][3], n = B * H * S * D;
    double *q = rnd(n), *k = rnd(n), *v = rnd(n), *d = rnd(n);
    double *o = (double*)malloc(sizeof(double) * n), *l = (double*)malloc(sizeof(double) * B * H * S);
    double *dq = (double*)malloc(sizeof(double) * n), *dk = (double*)malloc(sizeof(double) * n), *dv = (double*)malloc(sizeof(double) * n);
    for (int c = 0; c < 2; ++c) {
      if (oracle_attn_fwd(q, k, v, B, H, S, D, 0.3, c, o, l)) return 10;
      if (oracle_attn_bwd(q, k, v, d, B, H, S, D, 0.3, c, dq, dk, dv)) return 11;
      if (oracle_attn_bwd_head(q, k, v, d, S, D, 0.3, c, dq, dk, dv, o, l)) return 12;
      long pos[3] = {0, S / 2, S - 1};
      double* qr = rnd(3 * D);
      double *orow = (double*)malloc(sizeof(double) * 3 * D), lrow[3];
      if (oracle_attn_fwd_rows(qr, pos, 3, k, v, S, D, 0.3, c, orow, lrow)) return 13;
      free(qr); free(orow);
    }
    for (long m = 1; m <= S; m += (S > 2 ? S - 1 : 1))
      if (oracle_attn_bwd_causal_tail(q + (S - m) * D, d + (S - m) * D, m, k, v, S, D, 0.3, dq, dk, dv)) return 14;
    free(q); free(k); free(v); free(d); free(o); free(l); free(dq); free(dk); free(dv);
  }
  double x[4] = {0}, y[4] = {0};
  long bad[1] = {5};
  if (oracle_attn_fwd(x, x, x, 0, 1, 1, 1, 1.0, 0, y, y) != -1) return 20;
  if (oracle_attn_fwd_rows(x, bad, 1, x, x, 2, 2, 1.0, 0, y, y) != -1) return 21;
  if (oracle_attn_bwd_causal_tail(x, x, 3, x, x, 2, 2, 1.0, y, y, y) != -1) return 22;
  if (oracle_attn_bwd_head(x, x, x, x, 0, 2, 1.0, 0, y, y, y, 0, 0) != -1) return 23;
  puts("oracle ok");
  return 0;
}
"""

STUB = r"""
#include "attn_internal.h"
namespace attn {
int g_launches = 0;
hipError_t launch_fwd(const FwdParams& p, int, bool, int, hipStream_t) {
  ++g_launches;
  return p.bh > 0 && p.c > 0.0f ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_fwd_counting(const FwdParams&, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd(const BwdParams& p, int, bool, unsigned, hipStream_t) {
  ++g_launches;
  return p.nblk > 0 ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_bwd_dq(const BwdParams&, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fwd_short(const FwdParams&, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int, bool, hipStream_t) {
  ++g_launches;
  return p.vscale > 0.0f ? hipSuccess : hipErrorInvalidValue;
}
}
extern "C" int stub_launches(void) { return attn::g_launches; }
extern "C" int stub_xcd_group(int hpx, long kv_bytes) { return attn::xcd_group(hpx, kv_bytes); }
"""

ABI_DRIVER = r"""
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include "attn.h"
int stub_launches(void);
int stub_xcd_group(int hpx, long kv_bytes);
#define P ((void*)(uintptr_t)0x10000)
#define F ((float*)(uintptr_t)0x10000)
#define CHECK(expr, want) do { int r_ = (expr); if (r_ != (want)) { \
  printf("line %d: %s = %d, want %d\n", __LINE__, #expr, r_, (want)); return 1; } } while (0)
int main(void) {
  const int dims[] = {1, 2, 7, 64, 128, 129, 255, 256, 257, 65535, 1 << 20, INT_MAX, -1, 0, INT_MIN};
  const int nd = sizeof(dims) / sizeof(dims[0]);
  /* every shape combination through every validation path (misaligned v, so
     no valid shape reaches a launch): never UB, never a crash */
  for (int a = 0; a < nd; ++a)
    for (int b = 0; b < nd; ++b)
      for (int c = 0; c < nd; ++c)
        for (int D = 32; D <= 160; D += 32) {
          int r = attn_fwd(P, P, (char*)P + 8, P, F, dims[a], dims[b], dims[c], D, 0.1f, 1, 0);
          if (r == 0 || r == 8) { printf("shape passed validation with a misaligned pointer\n"); return 1; }
          (void)attn_bwd_workspace_size(dims[a], dims[b], dims[c], D);
          r = attn_bwd(P, P, P, P, F, P, P, P, P, 0, 0, dims[a], dims[b], dims[c], D, 0.1f, 1, 0);
          if (r != 1) { printf("bwd with a null workspace returned %d\n", r); return 1; }
          r = attn_fwd_fp8(P, P, P, P, F, dims[a], dims[b], dims[c], D, 0.1f, 0, 1.0f, 1.0f, 0.0f, 0);
          if (r == 0) { printf("fp8 with a zero descale passed\n"); return 1; }
        }
  CHECK(attn_fwd(0, P, P, P, F, 1, 1, 16, 128, 0.1f, 0, 0), 1);
  CHECK(attn_fwd(P, P, P, P, F, 1, 1, 16, 96, 0.1f, 0, 0), 3);
  CHECK(attn_fwd(P, P, P, P, F, 1, 1 << 23, 1, 64, 0.1f, 0, 0), 2);
  CHECK(attn_fwd(P, P, P, P, F, 1, 1, 16, 128, 3.0e38f, 0, 0), 6);
  CHECK(attn_fwd_ex(P, P, P, P, F, 1, 1, 300, 128, 0.1f, 1, 65.0f, 0), 6);
  CHECK(attn_fwd_policy(P, P, P, P, F, 1, 1, 300, 128, 0.1f, 1, 8.0f, 5, 0), 7);
  float tau; int poly;
  CHECK(attn_fwd_default_policy(128, 1, 8192, &tau, &poly), 0);
  CHECK(attn_fwd_default_policy(128, 1, 8192, 0, &poly), 1);
  CHECK(attn_fwd_rescale_events(P, P, P, P, F, 1, 1, 300, 128, 0.1f, 1, 8.0f, 0, 0), 1);
  CHECK(attn_fwd_fp8(P, P, P, P, F, 1, 1, 300, 128, 1e30f, 1, 1e30f, 1.0f, 1.0f, 0), 6);
  CHECK(attn_bwd_phases(P, P, P, P, F, P, P, P, P, P, 1024, 1, 1, 16, 128, 0.1f, 1, 8, 0), 7);
  CHECK(attn_bwd(P, P, P, P, F, P, P, P, P, P, 511, 1, 1, 16, 128, 0.1f, 1, 0), 5);
  CHECK(attn_bwd_noalloc(P, P, P, P, F, P, P, P, P, 1, 32, 65537, 128, 0.1f, 1, 0), 9);
  CHECK(attn_bwd_noalloc(0, P, P, P, F, P, P, P, P, 1, 1, 16, 128, 0.1f, 1, 0), 1);
  for (int s = -3; s < 12; ++s)
    if (!attn_strerror(s)) return 1;
  (void)attn_last_hip_error();
  CHECK(attn_version() >= 100, 1);
  /* valid requests reach the (stub) launch */
  const int before = stub_launches();
  CHECK(attn_fwd(P, P, P, P, F, 2, 3, 300, 128, -0.2f, 1, 0), 0);
  CHECK(attn_fwd(P, P, P, P, F, 2, 3, 100, 64, 0.0f, 0, 0), 0);
  CHECK(attn_fwd_ex(P, P, P, P, F, 1, 1, 300, 128, 0.1f, 1, 64.0f, 0), 0);
  CHECK(attn_fwd_policy(P, P, P, P, F, 1, 1, 300, 128, 0.1f, 1, 8.0f, 4, 0), 0);
  CHECK(attn_fwd_rescale_events(P, P, P, P, F, 1, 1, 300, 128, 0.1f, 1, 8.0f, (unsigned long long*)P, 0), 0);
  CHECK(attn_fwd_fp8(P, P, P, P, F, 1, 1, 300, 128, 0.1f, 1, 0.5f, 0.25f, 2.0f, 0), 0);
  CHECK(attn_bwd(P, P, P, P, F, P, P, P, P, P, attn_bwd_workspace_size(1, 1, 300, 128), 1, 1, 300, 128, 0.1f, 1, 0), 0);
  CHECK(attn_bwd_phases(P, P, P, P, F, P, P, P, P, P, 8192, 1, 1, 300, 128, 0.1f, 0, 3, 0), 0);
  CHECK(stub_launches() - before, 8);
  /* causal head groups per XCD: the largest divisor of the XCD's heads whose
     K/V fits 8 MiB, at least two (or all heads when no such divisor exists) */
  const long MiB = 1L << 20;
  CHECK(stub_xcd_group(0, MiB), 1);
  CHECK(stub_xcd_group(1, 64 * MiB), 1);
  CHECK(stub_xcd_group(2, 64 * MiB), 2);
  CHECK(stub_xcd_group(4, 2 * MiB), 4);    /* bf16, S = 4096, 32 heads */
  CHECK(stub_xcd_group(8, 4 * MiB), 2);    /* bf16, S = 8192, 64 heads */
  CHECK(stub_xcd_group(8, 2 * MiB), 4);    /* E4M3, S = 8192, 64 heads */
  CHECK(stub_xcd_group(12, MiB), 6);
  CHECK(stub_xcd_group(9, 4 * MiB), 9);    /* no divisor fits: all at once */
  CHECK(stub_xcd_group(6, 8 * MiB), 2);
  puts("abi ok");
  return 0;
}
"""


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    drv = tmp_path / "drv.c"
    drv.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_san"
    _run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-std=c11", str(drv), os.path.join(ROOT, "oracle", "oracle.c"),
          "-o", str(exe), "-lm"])
    r = _run([str(exe)], env=ENV, timeout=300)
    assert "oracle ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_host_layer_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "exact_attention_128_amd", "csrc")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + csrc]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-fno-gpu-sanitize"]
    base = [HIPCC, "-std=c++20", "-O1", "-g", "--offload-arch=gfx950", "-Xclang", "-target-feature",
            "-Xclang", "-packed-fp32-ops"]
    objs = []
    for name in ("attn_api.hip", "attn_noalloc.hip"):
        obj = str(tmp_path / (name + ".o"))
        _run(base + san + inc + ["-c", os.path.join(csrc, name), "-o", obj])
        objs.append(obj)
    (tmp_path / "stub.hip").write_text(STUB)
    _run(base + san + inc + ["-c", str(tmp_path / "stub.hip"), "-o", str(tmp_path / "stub.o")])
    (tmp_path / "drv.c").write_text(ABI_DRIVER)
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I" + os.path.join(ROOT, "include"), "-c", str(tmp_path / "drv.c"), "-o",
          str(tmp_path / "drv.o")])
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-fno-gpu-sanitize"] + objs +
         [str(tmp_path / "stub.o"), str(tmp_path / "drv.o"), "-o", exe])
    r = _run([exe], env=ENV, timeout=600)
    assert "abi ok" in r.stdout
