// attn_fwd_short.hip -- exact-attention forward for short sequences (S <= 128)
// on gfx950 (MI355X).
//
// Same result as attn_fwd.hip (O = softmax(scale * Q K^T [causal]) V and the
// natural-log LSE), for the latency- and HBM-bound corner of the roofline
// (Tencent Cloud article "AI Infra 系列 第六章 GPU 性能工程（二）", section 2:
// at a few MFLOP per head the time is load latency, not matrix work).  With at
// most 128 keys a whole row of scores fits in registers, so:
//   * one burst of loads: every wave issues its Q rows (to registers) and its
//     share of the head's K and V (HBM -> LDS directly), then one wait and one
//     barrier -- a single HBM round trip before any arithmetic;
//   * one-pass softmax with the exact row maximum (no online rescaling, no
//     second pass): m = max_j s_ij, P = exp2(s c - m c), then the PV product;
//   * 4 waves x 32 query rows per workgroup (no ping-pong), packed by
//     sequence length so that no wave idles: one head of up to 128 rows, two
//     heads of up to 64 rows, or four heads of up to 32 rows per workgroup
//     (the memory-bound side of the roofline, [Tencent, section 2]: many
//     small heads, each a few KiB of HBM traffic).  A head keeps only the K/V
//     rows it can have in LDS -- two 64-key sub-tiles for up to 128 keys, one
//     for up to 64, one of 32 keys for up to 32 -- so the LDS a head holds,
//     which bounds the heads in flight per CU, shrinks with the sequence.
// The products, fragment layouts and row sums are those of the long-sequence
// kernel: S^T = K Q^T (32x32x16 bf16 MFMA, A = K from LDS, B = Q in
// registers, one query row per lane), O^T += V^T P^T with V^T read by the
// transposing LDS load and P straight from registers, O normalised by the sum
// of the bf16-rounded P the product consumes, LSE from the fp32 sum.
#include "attn_internal.h"
#include "gfx950.h"

namespace attn {

// WPH waves (32 query rows each) per head, 4 / WPH heads per workgroup; a head
// has at most 32 * WPH keys, held as NSUB sub-tiles of BC keys of K and V in
// LDS (BC = 32 when WPH = 1, else 64).
template <int D, bool CAUSAL, int WPH>
__global__ __launch_bounds__(256) void attn_fwd_short_kernel(FwdParams p) {
  constexpr int NW = 4;
  constexpr int HPW = NW / WPH;        // heads per workgroup
  constexpr int NSUB = WPH == 4 ? 2 : 1;
  constexpr int BC = WPH == 1 ? 32 : 64;
  constexpr int NG = BC / 16;          // 16-key groups per sub-tile
  constexpr int KB = BC / 32;          // 32-key blocks per sub-tile
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int CH = D / 8;
  constexpr int KSUB = CH * BC * 16;   // K sub-tile [CH][BC keys][16 B]
  constexpr int VSUB = DB * BC * 64;   // V sub-tile [DB][BC keys][64 B]
  constexpr int HLDS = NSUB * (KSUB + VSUB);   // one head's K and V
  constexpr int NKB = WPH;             // 32-key blocks that can hold a key
  // 1 KiB pieces of one DMA instruction each: K (sub-tile, chunk column) for
  // 64-key sub-tiles, two adjacent chunk columns for 32-key ones; V
  // (sub-tile, feature block, 16-key group)
  constexpr int KPIECE = NSUB * CH * BC / 64;
  constexpr int VPIECE = NSUB * DB * NG;
  static_assert(NW % WPH == 0 && NKB <= 2 * NSUB, "a head's waves and keys must fit");
  static_assert(KPIECE % WPH == 0 && VPIECE % WPH == 0, "pieces must split over a head's waves");

  __shared__ __attribute__((aligned(16))) char smem[HPW * HLDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = w / WPH;              // head slot of this wave
  const int wi = w % WPH;              // wave within the head
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int S = p.S;

  // the head of this wave; a slot past the last head loads nothing and ends
  // after the barrier
  const long bhl = (long)blockIdx.x * HPW + hs;
  const bool live = bhl < p.bh;
  const int bh = live ? (int)bhl : p.bh - 1;
  const int qw = 32 * wi;
  const int qrow = qw + l32;
  const size_t head = (size_t)bh * S * D;

  // ---- the burst: K and V of the head into LDS (rows past S read as zero),
  //      split over the head's waves, then this lane's Q row
  const uint32_t hbytes = (uint32_t)S * D * 2;
  const uint16_t* const Kh = p.k + head;
  const uint16_t* const Vh = p.v + head;
  ATTN_LDS char* const ks = (ATTN_LDS char*)smem + hs * HLDS;
  ATTN_LDS char* const vs = ks + NSUB * KSUB;
  if (live) {
#pragma unroll
    for (int k = 0; k < KPIECE / WPH; ++k) {
      const int i = wi + WPH * k;
      if constexpr (BC == 64) {
        const int st = i / CH, cc = i % CH;
        const u32x4 rs = buffer_rsrc_at(Kh, hbytes, (uint32_t)(st * BC) * (2 * D));
        lds_dma16(ks + st * KSUB + cc * 1024, rs, lane * (2 * D), cc * 16);
      } else {
        // lanes 0-31: key l32 of chunk column 2i, lanes 32-63: of column 2i+1
        const u32x4 rs = buffer_rsrc_at(Kh, hbytes, 0u);
        lds_dma16(ks + i * 1024, rs, l32 * (2 * D) + h * 16, i * 32);
      }
    }
    const int vl_off = (lane >> 2) * (2 * D) + (lane & 3) * 16;
#pragma unroll
    for (int k = 0; k < VPIECE / WPH; ++k) {
      const int i = wi + WPH * k;
      const int st = i / (DB * NG), r = i % (DB * NG), db = r / NG, rg = r % NG;
      const u32x4 rs = buffer_rsrc_at(Vh, hbytes, (uint32_t)(st * BC + 16 * rg) * (2 * D));
      lds_dma16(vs + st * VSUB + db * (BC * 64) + rg * 1024, rs, vl_off, db * 64);
    }
  }
  bf16x8 qf[KK];
  {
    const bool ok = live && qrow < S;
    const uint16_t* qr = p.q + head + (size_t)(ok ? qrow : S - 1) * D + 8 * h;
    const uint32_t qm = ok ? p.qand : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = *(const u32x4*)(qr + 16 * kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (x[e] ^ p.qxor) & qm;
      qf[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }
  wait_vmcnt<0>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // a wave with no head or no valid row (after the barrier: its loads are in)
  if (!live || qw >= S) return;

  // ---- S^T = K Q^T over every key; s[b] = 32-key block b (key 32b + 8(r/4) +
  //      4h + r%4 of register r, query qrow)
  f32x16 s[NKB];
  const int kbase = h * (BC * 16) + l32 * 16;
#pragma unroll
  for (int b = 0; b < NKB; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[b][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 a = lds_read_b128(ks + (b / KB) * KSUB + 2 * kk * (BC * 16) + 32 * (b % KB) * 16 +
                                     kbase);
      s[b] = mfma32(a, qf[kk], s[b]);
    }
  }
  // keys past S, and above the diagonal, get -inf
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < NKB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
      if (!(key < S && (!CAUSAL || key <= qrow))) s[b][r] = -INFINITY;
      mx = fmaxf(mx, s[b][r]);
    }
  mx = halfwave_max(mx);
  // every row sees key 0 (causal: key 0 <= qrow), so mx is finite
  const float c = p.c;
  const float m = mx * c;   // the exact row maximum, log2 units
  float lf = 0.0f, lb = 0.0f;
  uint32_t pk[NKB][8];
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
  for (int b = 0; b < NKB; ++b) {
    f32x16 e;
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, -m));
#pragma unroll
    for (int r = 0; r < 16; ++r) lf += e[r];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pk[b][j] = pack_bf16x2(e[2 * j], e[2 * j + 1]);
      lb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[b][j]), one, lb, false);
    }
  }

  // ---- O^T += V^T P^T over every 16-key group g (sub-tile g/NG, group g%NG)
  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  const int vbase = (4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * 64 +
                    (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
#pragma unroll
  for (int g = 0; g < 2 * NKB; ++g) {
    const uint32_t* pp = &pk[g >> 1][4 * (g & 1)];
    const u32x4 pw = {pp[0], pp[1], pp[2], pp[3]};
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const ATTN_LDS char* rb = vs + vbase + (g / NG) * VSUB + 16 * (g % NG) * 64 + db * (BC * 64);
      const u32x2 a0 = __builtin_bit_cast(u32x2, lds_read_tr16(rb));
      const u32x2 a1 = __builtin_bit_cast(u32x2, lds_read_tr16(rb + 8 * 64));
      const u32x4 aw = {a0[0], a0[1], a1[0], a1[1]};
      o[db] = mfma32(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, pw), o[db]);
    }
  }

  // ---- epilogue: O = O / l_b (bf16), LSE = ln2 * (m + log2 l_f)
  lf = halfwave_sum(lf);
  lb = halfwave_sum(lb);
  if (qrow < S) {
    const float inv = 1.0f / lb;
    uint16_t* orow = p.o + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * h;
        const u32x2 wv = {pack_bf16x2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                          pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
        *(u32x2*)(orow + d) = wv;
      }
    if (h == 0) p.lse[(size_t)bh * S + qrow] = (m + __builtin_amdgcn_logf(lf)) * kLn2;
  }
}

template <int D, bool CAUSAL, int WPH>
static hipError_t launch_short_t(const FwdParams& p, hipStream_t stream) {
  constexpr int HPW = 4 / WPH;
  const long grid = ((long)p.bh + HPW - 1) / HPW;
  if (p.bh <= 0 || grid * 256 > 0xffffffffL) return hipErrorInvalidConfiguration;
  FwdParams pp = p;
  void* args[] = {&pp};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_short_kernel<D, CAUSAL, WPH>),
                         dim3((unsigned)grid), dim3(256), args, 0, stream);
}

template <int D, bool CAUSAL>
static hipError_t launch_short_d(const FwdParams& p, hipStream_t stream) {
  if (p.S <= 32) return launch_short_t<D, CAUSAL, 1>(p, stream);
  if (p.S <= 64) return launch_short_t<D, CAUSAL, 2>(p, stream);
  return launch_short_t<D, CAUSAL, 4>(p, stream);
}

hipError_t launch_fwd_short(const FwdParams& p, int D, bool causal, hipStream_t stream) {
  static_assert(kShortMaxS <= 4 * 32, "four waves of 32 rows hold every query row of a head");
  if (p.S < 1 || p.S > kShortMaxS) return hipErrorInvalidValue;
  if (D == 128) return causal ? launch_short_d<128, true>(p, stream) : launch_short_d<128, false>(p, stream);
  if (D == 64) return causal ? launch_short_d<64, true>(p, stream) : launch_short_d<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
