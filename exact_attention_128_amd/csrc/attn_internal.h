// attn_internal.h -- launch descriptors shared by the host entry points and
// the kernel translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr float kLog2eHost = 1.4426950408889634f;

// One forward launch.  Tensors are [B*H][S][D] bf16 (raw 16-bit words).
struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int bh;         // B * H
  int S;          // sequence length (queries = keys)
  int nqb;        // query blocks per head
  float c;        // |scale| * log2(e), or 1 when scale == 0 (always > 0)
  uint32_t qxor;  // applied to every Q word pair: 0 (scale > 0) or 0x80008000 (scale < 0)
  uint32_t qand;  // 0xffffffff, or 0 when scale == 0 (Q treated as zero)
  float tau;      // rescale threshold in log2 units
  float thresh;   // 2^tau: a lane's partial weight sum above it triggers a rescale
  int xcd_heads;  // heads per XCD for the XCD-aware block order, 0 = plain order
  int xcd_group;  // causal: an XCD works through its heads this many at a time
                  // (divides xcd_heads; = xcd_heads: all at once)
  unsigned long long* events;  // diagnostic counters (see attn_fwd_rescale_events), or null
};

// One FP8 forward launch.  Q, K, V are [B*H][S][D] E4M3 codes (one byte per
// element); the scores are (Q codes . K codes) * c with c = |scale * q_descale
// * k_descale| * log2(e); O is bf16 and carries v_descale.
struct Fp8FwdParams {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  int bh;
  int S;
  int nqb;
  float c;        // > 0
  float vscale;   // v_descale, applied to O
  uint32_t qxor;  // 0, or 0x80808080 when scale < 0
  uint32_t qand;  // 0xffffffff, or 0 when scale == 0
  int xcd_heads;
  int xcd_group;  // causal: an XCD works through its heads this many at a time
};

// Causal XCD-aware block order: how many of an XCD's hpx heads it works on at
// a time.  The largest divisor of hpx whose K/V (kv_bytes per head) stays
// within 8 MiB, two L2s' worth, but at least two heads: with one head at a
// time the heaviest blocks of each head start late and the tail grows
// (measured: +28 % on 32 heads of S = 4096).  Measured on 64 heads of S = 8192
// (4 MiB of bf16 K/V each, groups of 2 against all 8 of an XCD's heads at
// once): 58 % less HBM read, -1.6 to -2.2 % time, the same bits.
inline int xcd_group(int hpx, long kv_bytes) {
  if (hpx <= 2) return hpx > 0 ? hpx : 1;
  int g = hpx;
  while (g > 2 && (g * kv_bytes > (8L << 20) || hpx % g != 0)) --g;
  return hpx % g == 0 ? g : hpx;
}

// One backward launch.
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* stats;  // workspace [B*H][nblk * 64 rows][8] bf16: per query row the
                    // record of -LSE*log2(e) and -Delta (stat_record in gfx950.h;
                    // zero for the rows past S in the last 64-row block)
  int bh;
  int S;
  int nblk;       // 64-row blocks per head, ceil(S / 64)
  int nqb;        // query blocks per head of the dQ kernel
  float scale;    // the logit scale (any finite value)
  float c;        // scale * log2(e)
  float cq;       // |scale| * log2(e), or 1 when scale == 0 (always > 0); the dQ
                  // kernel scores Q' K with Q' = Q with the sign of scale folded in:
  uint32_t qxor;  //   applied to every Q word pair: 0, or 0x80008000 when scale < 0
  uint32_t qand;  //   0xffffffff, or 0 when scale == 0 (Q' = 0)
  int xcd_heads;  // heads per XCD for the XCD-aware block order, 0 = plain order
  int xcd_group;  // dQ kernel, causal: an XCD works through its heads this many
                  // at a time (set by its launcher; the dK/dV kernel takes all)
};

// ATTN_OK for hipSuccess; otherwise records e as the calling thread's last HIP
// error (attn_last_hip_error) and returns ATTN_ERR_HIP.
int hip_status(hipError_t e);

// The backward's argument checks other than the workspace's; host only, no
// HIP call.  Returns ATTN_OK or an attn_status code.
int check_bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, const void* dq, const void* dk, const void* dv, int B,
                   int H, int S, int D, float scale);

// poly: the exponential policy of the long-sequence kernel (0, 4 or 8; see
// attn_fwd.hip); the short-sequence kernel always uses the hardware unit.
hipError_t launch_fwd(const FwdParams& p, int D, bool causal, int poly, hipStream_t stream);
hipError_t launch_fwd_counting(const FwdParams& p, int D, bool causal, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int D, bool causal, unsigned phases, hipStream_t stream);

// Sequences of at most kShortMaxS keys take the one-pass short-sequence
// forward (attn_fwd_short.hip): the whole row of scores in registers, exact
// row maxima, no conditional rescale.  (Measured: faster than the ping-pong
// kernel up to 128 keys -- 16.4 against 23.7 us for 320 causal heads of 128
// -- and slower at 256 keys, where the one-pass kernel's 128 KiB of LDS and
// one wave per SIMD leave the chip underused: 46 against 39 us.)
constexpr int kShortMaxS = 128;

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int D, bool causal, hipStream_t stream);
hipError_t launch_fwd_short(const FwdParams& p, int D, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, int D, bool causal, hipStream_t stream);

}  // namespace attn
