// attn_fwd.hip -- fused exact-attention forward for gfx950 (MI355X).
//
// Computes O = softmax(scale * Q K^T [causal]) V and the natural-log LSE per
// row in one kernel; the S x S scores live only in registers, one K/V tile at
// a time (the tiling and fusion levers of the Tencent Cloud article "AI Infra
// 系列 第六章 GPU 性能工程（二）", section 5; FA4's design in its section 7).
//
// Work decomposition.  A workgroup of NW = 8 waves owns BR = 256 consecutive
// query rows of one (batch, head); each wave owns 32 of them.  Waves w and
// w+4 share a SIMD.  The workgroup walks the key/value sequence in steps of
// 128 keys (two 64-key sub-tiles), K in a three-slot and V in a two-slot LDS
// ring.
//
// Each step of a wave has two halves:
//   matrix half   S^T = K Q^T for the NEXT step (4*D/16 MFMAs) and O^T +=
//                 V^T P^T for the CURRENT step (8*D/32 MFMAs), with their LDS
//                 fragment reads interleaved a few products ahead;
//   softmax half  the exponentials of the next tile's scores, their sums, and
//                 the bf16 packing of P.
// Waves 4..7 run half a step behind waves 0..3 (ping-pong, the portable form
// of FA4's overlap of tensor-core work with softmax work, Tencent Cloud
// article, section 7): on every SIMD one wave is in its matrix half, at
// raised issue priority, while the other wave's softmax arithmetic fills the
// issue slots the matrix core leaves free.  A workgroup barrier separates the
// half-steps.
//
//   S^T = K Q^T     32x32x16 bf16 MFMA; A = K rows from LDS, B = Q held in
//                   registers.  The transposed product puts one query row per
//                   lane (the two wave halves hold different keys of the same
//                   rows), so row statistics need one half-wave swap.
//   mask            only on the tile that crosses the causal diagonal or the
//                   sequence end; tiles wholly above a wave's diagonal are
//                   skipped by that wave.
//   online softmax  FA4's conditional rescaling (Tencent Cloud article, section
//                   7: rescale only when the running maximum moves enough to
//                   threaten the number range).  A row's first tile sets its
//                   maximum m exactly; later tiles are exponentiated straight
//                   against the stale m, with no per-tile maximum at all.  If
//                   any lane's partial sum of the new weights exceeds 2^tau
//                   (which happens whenever some score passed m by more than
//                   tau, in log2 units, and catches an overflow to inf), the
//                   wave moves each row's m up to that row's new maximum,
//                   rescales O and the sums, and redoes the tile's
//                   exponentials from the kept exponents.  The stale m cancels
//                   between numerator and denominator, so the result is exact.
//   P = exp2(S c - m) on the hardware exp unit (v_exp_f32).  On gfx950 it
//                   shares the VALU issue port and costs about three FMAs, so
//                   FA4's polynomial exp2 on the FMA pipe (Cody-Waite + cubic,
//                   section 7) would cost more issue slots than it frees.
//   O^T += V^T P^T  32x32x16 bf16 MFMA; B = P straight from registers (bf16),
//                   A = V^T fragments read with the transposing LDS load.
//
// K/V tiles travel from HBM straight into LDS (buffer loads with the LDS
// destination bit: no staging registers, no LDS write instructions), K three
// and V two steps ahead of use.  The LDS tiles use blocked layouts in which every
// fragment read (and every tile write) is a contiguous 256-byte run per 16 or
// 32 lanes -- free of bank conflicts (the conflict-avoidance lever of the
// Tencent Cloud article, section 4) without swizzling -- and each lane reaches
// all of its fragments at fixed offsets from one base address:
//   K  [D/8 chunk columns][64 keys][16 bytes]
//   V  [D/32 feature blocks][64 keys][32 features]
//
// Two row sums: O is normalised by the sum of the bf16-rounded P that the PV
// product consumes (so the weights of O sum to one exactly in the products'
// own rounding), the LSE takes the fp32 sum of P.
#include "attn_internal.h"
#include "gfx950.h"

namespace attn {

template <int D>
struct FwdTile {
  static constexpr int BC = 64;               // keys per sub-tile
  static constexpr int CH = D / 8;            // 16-byte chunk columns of a K row
  static constexpr int DB = D / 32;           // 32-feature blocks of a V row
  static constexpr int KSUB = CH * BC * 16;   // K sub-tile [CH][64 keys][16 B]
  static constexpr int VSUB = DB * BC * 64;   // V sub-tile [DB][64 keys][64 B]
  static constexpr int KSLOT = 2 * KSUB;      // a step's 128 keys
  static constexpr int VSLOT = 2 * VSUB;
  static constexpr int NKS = 3;               // K ring slots
  static constexpr int NVS = 2;               // V ring slots
  static constexpr int LDS = NKS * KSLOT + NVS * VSLOT;
  // 1 KiB pieces per step: K one per (sub-tile, chunk column), V one per
  // (sub-tile, feature block, 16-key group); each group of 4 waves moves one.
  static constexpr int KPIECE = 2 * CH;
  static constexpr int VPIECE = 2 * DB * (BC / 16);
};

// FA4's software exponential (Tencent Cloud article, section 7: Cody-Waite
// range reduction and a cubic on the FMA units, for a share of the
// elements).  In base 2 the range reduction is exact: x = n + f with
// n = floor(x), f in [0, 1); 2^f is a cubic fitted here for minimax relative
// error on [0, 1) with p(0) = 1 exactly (so integer x give exact powers of
// two), max relative error 8.6e-5 -- 23 times below the 2^-9 rounding that P
// undergoes next; 2^n is applied by v_ldexp_f32.  The clamp sends -inf
// (masked keys) and anything below -160 to an exact 0 through ldexp's
// underflow; a finite x past 128 overflows to +inf exactly as v_exp_f32
// does, which the rescale test catches.
constexpr float kExpP1 = 0.6951172947883606f;
constexpr float kExpP2 = 0.22764353454113007f;
constexpr float kExpP3 = 0.077068030834198f;

__device__ __forceinline__ float exp2_poly(float x) {
  x = fmaxf(x, -160.0f);
  const float n = __builtin_floorf(x);
  const float f = x - n;
  const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(kExpP3, f, kExpP2), f, kExpP1), f,
                                 1.0f);
  return __builtin_ldexpf(p, (int)n);
}

// COUNT: the diagnostic instantiation behind attn_fwd_rescale_events, which
// also counts the rescale tests and the rescales (same arithmetic, same
// results; the production kernels are the COUNT = false ones).
// POLY: exponential policy -- 0: every exponential on the hardware unit
// (v_exp_f32); 4 or 8: every POLY-th exponential of a lane (a fixed column
// subset of each score tile, 25 % or 12.5 % of them) by exp2_poly instead.
template <int D, bool CAUSAL, bool COUNT = false, int POLY = 0>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p) {
  using T = FwdTile<D>;
  constexpr int NW = 8;
  constexpr int BR = 32 * NW;
  constexpr int BC = T::BC;
  constexpr int KK = D / 16;     // MFMA steps over the head dimension
  constexpr int DB = D / 32;     // 32-row blocks of O^T
  constexpr int CH = T::CH;
  constexpr int KPW = T::KPIECE / 4;   // K pieces per wave of the four that load a K tile
  constexpr int VPW = T::VPIECE / 4;   // V pieces per wave of the four that load a V tile
  static_assert(T::KPIECE % 4 == 0 && T::VPIECE % 4 == 0, "pieces must split over 4 waves");

  __shared__ __attribute__((aligned(16))) char smem[T::LDS];  // [K ring][V ring]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int grp = w >> 2;
  const int S = p.S;

  // ---- work unit: (head, query block).  Causal: heaviest query blocks first.
  //      With xcd_heads > 0, consecutive slots of one XCD (workgroup ids are
  //      dealt round-robin over the 8 XCDs) stay on the same heads, so their
  //      K/V re-reads hit that XCD's L2; causal, the XCD takes its heads
  //      xcd_group at a time (heaviest block first within the group).
  int bh, qi;
  {
    const int u = blockIdx.x;
    if (p.xcd_heads > 0) {
      const int x = u & 7, j = u >> 3;
      if (CAUSAL) {
        // the XCD's heads in groups of xcd_group, heaviest block first
        // within a group: a group's K/V fits the XCD's L2 far better than
        // all of its heads' at once
        const int G = p.xcd_group, per = G * p.nqb, gi = j / per, r = j % per;
        qi = r / G;
        bh = x + 8 * (gi * G + r % G);
      } else {
        bh = x + 8 * (j / p.nqb);
        qi = j % p.nqb;
      }
    } else {
      if (CAUSAL) {
        qi = u / p.bh;
        bh = u % p.bh;
      } else {
        bh = u / p.nqb;
        qi = u % p.nqb;
      }
    }
  }
  const int qb = CAUSAL ? p.nqb - 1 - qi : qi;
  const int q0 = qb * BR;
  const int qw = q0 + 32 * w;      // first row of this wave
  const int qrow = qw + l32;       // this lane's row
  const size_t head = (size_t)bh * S * D;
  const uint16_t* __restrict__ Qh = p.q + head;

  bf16x8 qf[KK];   // Q fragments, loaded in the prologue

  // keys [0, kend) matter to this workgroup, in steps of 2*BC; this wave uses
  // steps [0, wsteps)
  const int kend = CAUSAL ? min(S, q0 + BR) : S;
  const int nsteps = (kend + 2 * BC - 1) / (2 * BC);
  const int wend = CAUSAL ? min(S, qw + 32) : S;
  const int wsteps = qw < S ? (wend + 2 * BC - 1) / (2 * BC) : 0;

  // ---- K/V of a step: HBM -> LDS directly (rows past S read as zero), a
  //      tile split over the four waves of one group (one wave per SIMD; the
  //      schedule below says which group loads what).  Lane l of a K piece carries
  //      key l of one chunk column; lane l of a V piece carries 16 bytes of key
  //      l/4 of one feature block; every piece lands as one 1 KiB run.
  const uint32_t hbytes = (uint32_t)S * D * 2;
  const uint16_t* const Kh = p.k + head;
  const uint16_t* const Vh = p.v + head;
  const int kl_off = lane * (2 * D);
  const int vl_off = (lane >> 2) * (2 * D) + (lane & 3) * 16;
  ATTN_LDS char* const kring = (ATTN_LDS char*)smem;
  ATTN_LDS char* const vring = kring + T::NKS * T::KSLOT;
  auto fetch_k = [&](int st) {
    const int key0 = st * 2 * BC;
    ATTN_LDS char* base = kring + (st % T::NKS) * T::KSLOT;
#pragma unroll
    for (int k = 0; k < KPW; ++k) {
      const int i = (w & 3) + 4 * k;
      const int u = i / CH, cc = i % CH;
      const u32x4 rs = buffer_rsrc_at(Kh, hbytes, (uint32_t)(key0 + u * BC) * (2 * D));
      lds_dma16(base + u * T::KSUB + cc * 1024, rs, kl_off, cc * 16);
    }
  };
  auto fetch_v = [&](int st) {
    const int key0 = st * 2 * BC;
    ATTN_LDS char* base = vring + (st % T::NVS) * T::VSLOT;
#pragma unroll
    for (int k = 0; k < VPW; ++k) {
      const int i = (w & 3) + 4 * k;
      const int u = i / (DB * 4), r = i % (DB * 4), db = r >> 2, rg = r & 3;
      const u32x4 rs = buffer_rsrc_at(Vh, hbytes, (uint32_t)(key0 + u * BC + 16 * rg) * (2 * D));
      lds_dma16(base + u * T::VSUB + db * (BC * 64) + rg * 1024, rs, vl_off, db * 64);
    }
  };
  auto sync = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  int n_tests = 0, n_rescales = 0;   // COUNT only; wave-uniform
  float m_run = 0.0f;        // stale row max in log2 units (scores * c); set by step 0
  float l_f = 0.0f;          // sum of the fp32 weights: gives the LSE
  float l_b = 0.0f;          // sum of the weights rounded to bf16 (what the PV product
                             // consumes): normalises O
  const float c = p.c;
  const float thresh = p.thresh;   // 2^tau

  // Per-lane LDS byte offsets within a sub-tile; every fragment adds a constant.
  //   K (A operand of S^T): key 32b + l32, chunk column 2kk + h.
  //   V (transposing read, see lds_read_tr16): keys 16t + 4*half + tr_key
  //   (+8), features 32db + tr_d .. +3.
  const int kbase = h * (BC * 16) + l32 * 16;
  const int vbase = (4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * 64 +
                    (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  auto kslot = [&](int st) { return (const ATTN_LDS char*)kring + (st % T::NKS) * T::KSLOT; };
  auto vslot = [&](int st) { return (const ATTN_LDS char*)vring + (st % T::NVS) * T::VSLOT; };

  // S^T of step st's 128 keys: s[2u + b] = sub-tile u, 32-key block b
  auto qk = [&](int st, f32x16 (&s)[4]) {
    const ATTN_LDS char* kb = kslot(st) + kbase;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const bf16x8 a = lds_read_b128(kb + u * T::KSUB + 2 * kk * (BC * 16) + 32 * b * 16);
          s[2 * u + b] = mfma32(a, qf[kk], s[2 * u + b]);
        }
  };
  // The matrix half: S^T of step ks and O^T += V^T P^T with the V of step
  // vs.  All fragment reads are written first and then interleaved with the
  // products by scheduling groups, so each product finds its operands LA
  // products ahead: LDS latency stays hidden without holding a whole tile in
  // registers.
  // K fragment i of a step (the A operand of score product i)
  auto kfrag = [&](const ATTN_LDS char* kb, int i) {
    const int u = i / (2 * KK), kk = (i % (2 * KK)) >> 1, b = i & 1;
    return lds_read_b128(kb + u * T::KSUB + 2 * kk * (BC * 16) + 32 * b * 16);
  };
  // The first LA K fragments of step st, read ahead of its matrix half (the
  // half then starts with a product instead of waiting out an LDS read).
  constexpr int LA = 5;
  auto kpre_read = [&](int st, bf16x8 (&kp)[LA]) {
    const ATTN_LDS char* kb = kslot(st) + kbase;
#pragma unroll
    for (int i = 0; i < LA; ++i) kp[i] = kfrag(kb, i);
  };
  auto mphase = [&](int ks, int vs, f32x16 (&s)[4], const uint32_t (&pk)[4][8],
                    const bf16x8 (&kp)[LA]) {
    constexpr int NQ = 4 * KK, NP = 8 * DB, NM = NQ + NP;
    const ATTN_LDS char* kb = kslot(ks) + kbase;
    const ATTN_LDS char* vb = vslot(vs) + vbase;
    bf16x8 kf[NQ];
    i16x4 vf[2 * NP];
#pragma unroll
    for (int i = 0; i < NQ; ++i) kf[i] = i < LA ? kp[i] : kfrag(kb, i);
#pragma unroll
    for (int bt = 0; bt < 8; ++bt)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const ATTN_LDS char* rb = vb + (bt >> 2) * T::VSUB + 16 * (bt & 3) * 64 + db * (BC * 64);
        vf[2 * (DB * bt + db)] = lds_read_tr16(rb);
        vf[2 * (DB * bt + db) + 1] = lds_read_tr16(rb + 8 * 64);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int u = i / (2 * KK), j = i % (2 * KK);
      s[2 * u + (j & 1)] = mfma32(kf[i], qf[j >> 1], s[2 * u + (j & 1)]);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int bt = i / DB, db = i % DB;   // 16-key group bt of the step's 128 keys
      const uint32_t* pp = &pk[bt >> 1][4 * (bt & 1)];
      const u32x4 pw = {pp[0], pp[1], pp[2], pp[3]};
      const u32x2 a0 = __builtin_bit_cast(u32x2, vf[2 * i]);
      const u32x2 a1 = __builtin_bit_cast(u32x2, vf[2 * i + 1]);
      const u32x4 aw = {a0[0], a0[1], a1[0], a1[1]};
      o[db] = mfma32(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, pw), o[db]);
    }
    MSched<NQ, NM, LA, true>::apply();
  };
  // keys past the sequence end, and above the causal diagonal, get -inf
  auto mask = [&](int st, f32x16 (&s)[4]) {
    const int key0 = st * 2 * BC;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        const bool vis = key < S && (!CAUSAL || key <= qrow);
        if (!vis) s[i][r] = -INFINITY;
      }
  };
  auto needs_mask = [&](int st) {
    const int key0 = st * 2 * BC;
    return (key0 + 2 * BC > S) || (CAUSAL && key0 + 2 * BC - 1 > qw);
  };
  auto row_max = [&](const f32x16 (&s)[4]) {
    float mx = s[0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[i][r]);
    return halfwave_max(mx);
  };
  // pack to bf16 (round to nearest even): the B operand of the PV product
  auto pack = [&](const f32x16 (&e)[4], uint32_t (&pk)[4][8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) pk[i][j] = pack_bf16x2(e[i][2 * j], e[i][2 * j + 1]);
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    l_f *= alpha;
    l_b *= alpha;
  };
  // e = 2^(x - mx) for the kept exponents x; returns this lane's partial sum.
  // All exponentials issue first and the sums follow behind a scheduling
  // barrier: an add right behind its v_exp_f32 would stall on the
  // transcendental's latency, which the compiler's schedule underestimates.
  auto expo = [&](const f32x16 (&x)[4], float mx, f32x16 (&e)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        e[i][r] = (POLY > 0 && r % (POLY > 0 ? POLY : 1) == 0) ? exp2_poly(x[i][r] - mx)
                                                                : __builtin_amdgcn_exp2f(x[i][r] - mx);
    __builtin_amdgcn_sched_barrier(0);
    float t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = e[k >> 1][8 * (k & 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((r & 7) != 0) t[2 * i + (r >> 3)] += e[i][r];
    return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
  };
  // this lane's sum of its packed bf16 weights (exact products by 1.0 in
  // v_dot2c_f32_bf16, fp32 accumulation), in four chains
  auto bsum = [&](const uint32_t (&pk)[4][8]) {
    const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3F803F80u);
    float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        t[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i][j]), one, t[i],
                                               false);
    return (t[0] + t[1]) + (t[2] + t[3]);
  };
  // Softmax of a later step against the stale maximum m, with conditional
  // rescaling.  x = s*c - m is kept until the weights e = 2^x have passed the
  // check, so the rare path needs no recomputation of the scores: it moves
  // each row's m up by its largest x (a row whose x never went positive keeps
  // m), scales O and the sums down to match, and redoes the exponentials.
  // Leaves the packed weights in pk.
  auto softmax = [&](f32x16 (&s)[4], uint32_t (&pk)[4][8]) {
    const float nm = -m_run;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = __builtin_fmaf(s[i][r], c, nm);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 e[4];
    float t = expo(s, 0.0f, e);
    if constexpr (COUNT) ++n_tests;
    if (wave_any(t > thresh)) {
      if constexpr (COUNT) ++n_rescales;
      const float mx = fmaxf(row_max(s), 0.0f);
      rescale(__builtin_amdgcn_exp2f(-mx));
      m_run += mx;
      t = expo(s, mx, e);
    }
    l_f += t;
    pack(e, pk);
    l_b += bsum(pk);
  };

  // ---- prologue.  Waves 4..7 request K of step 0 and every wave its Q rows;
  //      once they have landed (a full wait, so no load the compiler tracks is
  //      left pending), K of steps 1..2 and V of steps 0..1 are requested and
  //      stream in behind step 0's scores and softmax (the row maxima start
  //      exact).  Each wave then waits for its own pieces of K 1 (waves 4..7)
  //      or V 0 (waves 0..3), and a barrier makes them visible before the
  //      first reads of K 1.  K 2 and V 1 are waited for before the next
  //      barrier of their loading waves (below and at the end of the first
  //      matrix half), ahead of their first reads.
  if (grp == 1) fetch_k(0);
  // Q fragments (B operand of S^T = K Q^T): lane holds row qrow, features
  // 16*kk + 8*h .. +7 for step kk.  Branch-free: a lane past S loads the
  // last row and its mask zeroes the values, so the eight loads issue back
  // to back behind the K request.
  {
    const bool ok = qrow < S;
    const uint16_t* qr = Qh + (size_t)(ok ? qrow : S - 1) * D + 8 * h;
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
  sync();
  if (grp == 1) {
    if (nsteps > 1) fetch_k(1);
    if (nsteps > 2) fetch_k(2);
  } else {
    fetch_v(0);
    if (nsteps > 1) fetch_v(1);
  }

  uint32_t pk[4][8];
  if (wsteps > 0) {
    f32x16 s[4], e[4];
    qk(0, s);
    if (needs_mask(0)) mask(0, s);
    const float mx = row_max(s);
    m_run = mx == -INFINITY ? 0.0f : mx * c;   // every valid row sees key 0
    const float nm = -m_run;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = __builtin_fmaf(s[i][r], c, nm);
    l_f = expo(s, 0.0f, e);
    pack(e, pk);
    l_b = bsum(pk);
  }

  // ---- main loop over steps of 128 keys.  K of step j lives in K slot j % 3,
  //      V of step j in V slot j % 2.  Each wave's step j is its matrix half
  //      (S^T of step j+1, O^T += V^T P^T of step j), a barrier, its softmax
  //      half (step j+1) followed by the reads of the first K fragments of
  //      step j+2, and a barrier; waves 4..7 start one barrier late, so on
  //      every SIMD one wave's matrix half, at raised priority, meets the
  //      other's softmax half.  Global barriers 2j and 2j+1 close the matrix
  //      halves of step j of waves 0..3 and 4..7 (barrier -1 ends the
  //      prologue, by which K of step 1 and V of step 0 have landed; its
  //      loads of K of step 2 and V of step 1 are waited for before barrier
  //      0, ahead of their first reads after it).
  //      Loads are issued at the top of the softmax half, where the wave has
  //      time to spare, and waited for at the end of its next matrix half:
  //      waves 0..3 request K of step j+3 after barrier 2j (into the slot of
  //      K of step j, whose last reads end at barrier 2j-1) and wait before
  //      barrier 2j+2, the first reads of it coming after that barrier;
  //      waves 4..7 request V of step j+2 after barrier 2j+1 (into the slot of
  //      V of step j, whose last reads end at barrier 2j+1) and wait before
  //      barrier 2j+3, after which it is first read.  A wave at its last step
  //      still runs the score products of the (unused) next slot, so the
  //      matrix half has a single code path.
  if (grp == 1) {
    if (nsteps > 2) wait_vmcnt<KPW>();   // K 1 landed, K 2 may still be in flight
    else wait_vmcnt<0>();
  } else {
    if (nsteps > 1) wait_vmcnt<VPW>();   // V 0 landed, V 1 may still be in flight
    else wait_vmcnt<0>();
  }
  sync();
  bf16x8 kp[LA];
  kpre_read(1, kp);
  if (grp == 1) {
    wait_vmcnt<0>();   // K 2, read by waves 0..3 after this barrier
    sync();
  }
  for (int j = 0; j < nsteps; ++j) {
    f32x16 sn[4];
    if (j < wsteps) {
      __builtin_amdgcn_s_setprio(1);
      mphase(j + 1, j, sn, pk, kp);
      __builtin_amdgcn_s_setprio(0);
    }
    wait_vmcnt<0>();
    sync();
    if (grp == 0) {
      if (j + 3 < nsteps) fetch_k(j + 3);
    } else {
      if (j + 2 < nsteps) fetch_v(j + 2);
    }
    if (j + 1 < wsteps) {
      if (needs_mask(j + 1)) mask(j + 1, sn);
      softmax(sn, pk);
    }
    kpre_read(j + 2, kp);
    sync();
  }
  if (grp == 0) sync();

  // ---- epilogue: O = O / l_b (bf16), LSE = ln2 * (m + log2 l_f).  O is
  //      normalised by the sum of the same bf16-rounded weights its products
  //      used (a row dominated by one key then gets exactly that key's V,
  //      up to the output rounding); the LSE takes the fp32 sum, which the
  //      rounding of the weights would move by up to 2^-9 relative.
  const float lf = halfwave_sum(l_f);
  const float lb = halfwave_sum(l_b);
  if (qrow < S) {
    const float inv = 1.0f / lb;
    uint16_t* orow = p.o + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * h;
        u32x2 wv = {pack_bf16x2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                    pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
        *(u32x2*)(orow + d) = wv;
      }
    if (h == 0) p.lse[(size_t)bh * S + qrow] = (m_run + __builtin_amdgcn_logf(lf)) * kLn2;
  }
  if constexpr (COUNT) {
    if (lane == 0 && n_tests > 0) {
      atomicAdd(p.events, (unsigned long long)n_tests);
      atomicAdd(p.events + 1, (unsigned long long)n_rescales);
    }
  }
}

template <int D, bool CAUSAL, bool COUNT = false, int POLY = 0>
static hipError_t launch_fwd_t(const FwdParams& p0, hipStream_t stream) {
  constexpr int NW = 8;
  FwdParams p = p0;
  p.nqb = (p.S + 32 * NW - 1) / (32 * NW);
  p.xcd_heads = (p.bh % 8 == 0) ? p.bh / 8 : 0;
  p.xcd_group = xcd_group(p.xcd_heads, 4L * p.S * D);   // bf16 K and V of a head
  p.thresh = exp2f(p.tau);
  const long grid = (long)p.bh * p.nqb;
  if (grid <= 0 || grid * NW * 64 > 0xffffffffL) return hipErrorInvalidConfiguration;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<D, CAUSAL, COUNT, POLY>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, stream);
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_poly(const FwdParams& p, int poly, hipStream_t stream) {
  if (poly == 0) return launch_fwd_t<D, CAUSAL, false, 0>(p, stream);
  if (poly == 4) return launch_fwd_t<D, CAUSAL, false, 4>(p, stream);
  if (poly == 8) return launch_fwd_t<D, CAUSAL, false, 8>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdParams& p, int D, bool causal, int poly, hipStream_t stream) {
  if (p.S <= kShortMaxS) return launch_fwd_short(p, D, causal, stream);
  if (D == 128)
    return causal ? launch_fwd_poly<128, true>(p, poly, stream) : launch_fwd_poly<128, false>(p, poly, stream);
  if (D == 64)
    return causal ? launch_fwd_poly<64, true>(p, poly, stream) : launch_fwd_poly<64, false>(p, poly, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_counting(const FwdParams& p, int D, bool causal, hipStream_t stream) {
  if (!p.events) return hipErrorInvalidValue;
  // the one-pass short-sequence kernel makes no rescale test: nothing to count
  if (p.S <= kShortMaxS) return launch_fwd_short(p, D, causal, stream);
  if (D == 128)
    return causal ? launch_fwd_t<128, true, true>(p, stream) : launch_fwd_t<128, false, true>(p, stream);
  if (D == 64)
    return causal ? launch_fwd_t<64, true, true>(p, stream) : launch_fwd_t<64, false, true>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
