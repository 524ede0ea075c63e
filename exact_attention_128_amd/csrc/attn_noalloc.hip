// attn_noalloc.hip -- attn_bwd_noalloc: the backward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The backward's only scratch space is its row-statistics workspace (16
// bytes per query row of each head, rounded up to 64-row blocks).  Here it lives
// in a file-scope device array of kScratchBytes, one copy per GPU, held until
// the process ends.  The array's host-side name is a stand-in, not a device
// address: the device address comes from hipGetSymbolAddress, fetched once per
// device (with that device current) and kept per device, and only that
// address is ever handed to a kernel.
//
// Every call on one GPU shares that GPU's array and leaves the last call's
// statistics in it.  Nothing needs clearing: the dQ kernel writes every
// statistic the dK/dV kernel later reads, within the same call and on the same
// stream.  Calls that overlap on one GPU (two streams, or two host threads)
// race on the array.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return attn::hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return attn::hip_status(e);
      if (!p) return ATTN_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                     int H, int S, int D, float scale, int causal, attn_stream_t stream) {
  // every host-side check before the first HIP call
  int rc = attn::check_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, H, S, D, scale);
  if (rc) return rc;
  const size_t need = attn_bwd_workspace_size(B, H, S, D);
  if (need > kScratchBytes) return ATTN_ERR_SCRATCH;
  void* ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc) return rc;
  return attn_bwd_phases(q, k, v, o, lse, dout, dq, dk, dv, ws, kScratchBytes, B, H, S, D, scale,
                         causal, ATTN_BWD_ALL, stream);
}

}  // extern "C"
