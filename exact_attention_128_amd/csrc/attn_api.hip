// attn_api.hip -- the C ABI declared in include/attn.h: host-side argument
// validation, scale handling, workspace layout and dispatch to the kernels.
// Every check runs before the first HIP call, so invalid requests never touch
// the device.
#include <math.h>
#include <stdint.h>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace attn {

namespace {
thread_local int g_last_hip_error = 0;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  g_last_hip_error = static_cast<int>(e);
  return ATTN_ERR_HIP;
}

}  // namespace attn

namespace {

using attn::hip_status;

constexpr int64_t kMaxElems = int64_t(1) << 40;
// 256-row query blocks per launch: the forward and dQ kernels run one
// 512-thread workgroup per block on a 1-D grid, whose work-item count must
// stay below 2^32; the dK/dV kernel's 256-thread workgroups per 128-key block
// then stay below it too (ceil(S/128) <= 2 ceil(S/256)).
constexpr int64_t kMaxRowBlocks = int64_t(1) << 23;

int check_shape(int B, int H, int S, int D) {
  if (B < 1 || H < 1 || S < 1) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  const int64_t bh = int64_t(B) * H;
  if (bh > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  // the kernels address one head's [S][D] bf16 slab with 32-bit byte offsets;
  // checked first, it also keeps the element count below 2^31 * 2^29
  if (int64_t(S) * D >= (int64_t(1) << 29)) return ATTN_ERR_SHAPE;
  if (bh * (int64_t(S) * D) >= kMaxElems) return ATTN_ERR_SHAPE;
  if (bh * ((int64_t(S) + 255) / 256) >= kMaxRowBlocks) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// The kernels multiply each fp32 score by |scale| * log2(e); a scale whose
// product with log2(e) overflows fp32 would turn every weight into NaN.
bool scale_ok(float scale) { return isfinite(scale) && isfinite(fabsf(scale) * attn::kLog2eHost); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The forward's softmax policy for a shape: the rescale threshold tau (log2
// units) and the share of exponentials computed by the polynomial on the FMA
// pipe (poly: every poly-th of a lane, 0 = none) -- the two knobs FA4 tunes
// per hardware generation (Tencent Cloud article, section 7; QbitAI, "三招").
// The table holds the measured winner of a sweep of tau in {0, 8, 16, 32,
// 64} x poly in {0, 8, 4} over the four long forward workloads on MI355X
// (bench.py --sweep-policy): no polynomial share ever won (+2 to +8 % time:
// its eight VALU operations per element cost the softmax wave more issue
// slots than the transcendental unit frees), and tau = 64 was best or within
// 0.1 % of it on every workload (rising maxima: -0.9 % against tau = 32,
// -12 % against FA4's 8), so one setting serves every shape.  At tau = 64 a
// weight stays below 2^64 and a row's sums below 2^81, far inside fp32.
struct FwdPolicy {
  float tau;
  int poly;
};

FwdPolicy select_policy(int D, int causal, int S) {
  (void)D;
  (void)causal;
  (void)S;
  return FwdPolicy{64.0f, 0};
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int S, int D, float scale, int causal, float tau, int poly, attn_stream_t stream,
             unsigned long long* events = nullptr, bool counting = false) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (counting && !events) return ATTN_ERR_NULL;
  int rc = check_shape(B, H, S, D);
  if (rc) return rc;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return ATTN_ERR_ALIGN;
  if (counting && !aligned(events, 8)) return ATTN_ERR_ALIGN;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  if (!(tau >= 0.0f && tau <= 64.0f)) return ATTN_ERR_SCALE;
  if (poly != 0 && poly != 4 && poly != 8) return ATTN_ERR_UNSUPPORTED;
  if (counting && poly != 0) return ATTN_ERR_UNSUPPORTED;

  attn::FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.bh = B * H;
  p.S = S;
  // softmax(scale * q.k) == softmax(|scale| * (-q).k): negate Q (exact in
  // bf16) for a negative scale so the kernels always see c > 0; a zero scale
  // gives uniform weights, the same as zeroing Q.
  p.qand = 0xffffffffu;
  p.qxor = 0u;
  if (scale < 0.0f) p.qxor = 0x80008000u;
  if (scale == 0.0f) p.qand = 0u;
  p.c = (scale == 0.0f) ? 1.0f : fabsf(scale) * attn::kLog2eHost;
  p.tau = tau;
  p.events = events;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_status(counting ? attn::launch_fwd_counting(p, D, causal != 0, st)
                             : attn::launch_fwd(p, D, causal != 0, poly, st));
}

}  // namespace

namespace attn {

// The backward's argument checks other than the workspace's (null pointers,
// shape, alignment, scale), host-only.
int check_bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, const void* dq, const void* dk, const void* dv, int B,
                   int H, int S, int D, float scale) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
  int rc = check_shape(B, H, S, D);
  if (rc) return rc;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return ATTN_ERR_ALIGN;
  if (!scale_ok(scale)) return ATTN_ERR_SCALE;
  return ATTN_OK;
}

}  // namespace attn

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int S, int D, float scale, int causal, attn_stream_t stream) {
  const FwdPolicy pol = select_policy(D, causal, S);
  return fwd_impl(q, k, v, o, lse, B, H, S, D, scale, causal, pol.tau, pol.poly, stream);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S, int D, float scale, int causal, float rescale_log2,
                attn_stream_t stream) {
  const FwdPolicy pol = select_policy(D, causal, S);
  return fwd_impl(q, k, v, o, lse, B, H, S, D, scale, causal, rescale_log2, pol.poly, stream);
}

int attn_fwd_policy(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int S, int D, float scale, int causal, float rescale_log2,
                    int exp_poly_every, attn_stream_t stream) {
  return fwd_impl(q, k, v, o, lse, B, H, S, D, scale, causal, rescale_log2, exp_poly_every,
                  stream);
}

int attn_fwd_default_policy(int D, int causal, int S, float* rescale_log2, int* exp_poly_every) {
  if (!rescale_log2 || !exp_poly_every) return ATTN_ERR_NULL;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (S < 1) return ATTN_ERR_SHAPE;
  const FwdPolicy pol = select_policy(D, causal, S);
  *rescale_log2 = pol.tau;
  *exp_poly_every = pol.poly;
  return ATTN_OK;
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int S, int D, float scale, int causal, float q_descale, float k_descale,
                 float v_descale, attn_stream_t stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  int rc = check_shape(B, H, S, D);
  if (rc) return rc;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return ATTN_ERR_ALIGN;
  for (float d : {q_descale, k_descale, v_descale})
    if (!(isfinite(d) && d > 0.0f)) return ATTN_ERR_SCALE;
  const float sc = scale * q_descale * k_descale;
  if (!scale_ok(scale) || !scale_ok(sc)) return ATTN_ERR_SCALE;
  attn::Fp8FwdParams p{};
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.bh = B * H;
  p.S = S;
  // as the bf16 forward: a negative scale negates the Q codes (sign bit of
  // every byte), a zero scale zeroes them
  p.qxor = sc < 0.0f ? 0x80808080u : 0u;
  p.qand = sc == 0.0f ? 0u : 0xffffffffu;
  p.c = sc == 0.0f ? 1.0f : fabsf(sc) * attn::kLog2eHost;
  p.vscale = v_descale;
  return attn::hip_status(attn::launch_fwd_fp8(p, D, causal != 0,
                                               reinterpret_cast<hipStream_t>(stream)));
}

int attn_fwd_rescale_events(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int S, int D, float scale, int causal,
                            float rescale_log2, unsigned long long* events,
                            attn_stream_t stream) {
  return fwd_impl(q, k, v, o, lse, B, H, S, D, scale, causal, rescale_log2, 0, stream, events,
                  true);
}

size_t attn_bwd_workspace_size(int B, int H, int S, int D) {
  if (check_shape(B, H, S, D) != ATTN_OK) return 0;
  (void)D;
  const size_t stat_bytes = size_t(B) * H * ((S + 63) / 64) * 64 * 16;  // 16 B per row
  return round_up(stat_bytes, 256);
}

int attn_bwd_phases(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, int B, int H, int S, int D,
                    float scale, int causal, unsigned phases, attn_stream_t stream) {
  if (!workspace) return ATTN_ERR_NULL;   // null pointers first, as every entry point
  int rc = attn::check_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, H, S, D, scale);
  if (rc) return rc;
  if (!aligned(workspace, 256)) return ATTN_ERR_ALIGN;
  if (workspace_bytes < attn_bwd_workspace_size(B, H, S, D)) return ATTN_ERR_WORKSPACE;

  attn::BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.lse = lse;
  p.dout = static_cast<const uint16_t*>(dout);
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.nblk = (S + 63) / 64;
  p.stats = static_cast<uint16_t*>(workspace);
  p.bh = B * H;
  p.S = S;
  p.xcd_heads = (p.bh % 8 == 0) ? p.bh / 8 : 0;
  p.scale = scale;
  p.c = scale * attn::kLog2eHost;
  p.cq = scale == 0.0f ? 1.0f : fabsf(scale) * attn::kLog2eHost;
  p.qxor = scale < 0.0f ? 0x80008000u : 0u;
  p.qand = scale == 0.0f ? 0u : 0xffffffffu;
  if (phases == 0 || (phases & ~unsigned(ATTN_BWD_ALL)) != 0) return ATTN_ERR_UNSUPPORTED;
  return hip_status(
      attn::launch_bwd(p, D, causal != 0, phases, reinterpret_cast<hipStream_t>(stream)));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int H, int S, int D, float scale, int causal,
             attn_stream_t stream) {
  return attn_bwd_phases(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, S,
                         D, scale, causal, ATTN_BWD_ALL, stream);
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE:
      return "invalid shape: B, H, S >= 1, B*H*S*D < 2^40, S*D < 2^29, B*H*ceil(S/256) < 2^23";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension: D must be 64 or 128";
    case ATTN_ERR_ALIGN:
      return "misaligned pointer: bf16 tensors need 16 bytes, LSE 4, workspace 256";
    case ATTN_ERR_WORKSPACE: return "workspace smaller than attn_bwd_workspace_size()";
    case ATTN_ERR_SCALE:
      return "scale (or scale*log2(e)) not finite, or rescale threshold outside [0, 64]";
    case ATTN_ERR_UNSUPPORTED: return "request not supported by this build";
    case ATTN_ERR_HIP: return "HIP runtime error (see attn_last_hip_error)";
    case ATTN_ERR_SCRATCH:
      return "problem needs more scratch than the library's static buffer holds "
             "(attn_bwd_noalloc: attn_bwd_workspace_size() must not exceed "
             "attn_noalloc_scratch_bytes())";
    default: return "unknown status code";
  }
}

int attn_last_hip_error(void) { return attn::g_last_hip_error; }

int attn_version(void) { return 100; }

}  // extern "C"
