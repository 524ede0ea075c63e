// attn_fwd.hip -- fused exact-attention forward for gfx950 (MI355X).
//
// Computes O = softmax(scale * Q K^T [causal]) V and the natural-log LSE per
// row in one kernel; the S x S scores live only in registers, one K/V tile at
// a time (the tiling and fusion levers of the Tencent Cloud article "AI Infra
// 系列 第六章 GPU 性能工程（二）", section 5; FA4's design in its section 7).
//
// Work decomposition.  A workgroup of NW = 8 waves owns BR = 256 consecutive
// query rows of one (batch, head); each wave owns 32 of them.  Waves w and
// w+4 share a SIMD.  The workgroup walks the key/value sequence in tiles of
// BC = 64 keys held in a four-slot LDS ring.
//
// Each tile step of a wave has two halves:
//   matrix half   S^T = K Q^T for the NEXT tile (16 MFMAs) and O^T += V^T P^T
//                 for the CURRENT tile (4*D/32 MFMAs), with their LDS fragment
//                 reads interleaved a few products ahead;
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
// destination bit: no staging registers, no LDS write instructions), three
// tiles ahead of use.  The LDS tiles use blocked layouts in which every
// fragment read (and every tile write) is a contiguous 256-byte run per 16 or
// 32 lanes -- free of bank conflicts (the conflict-avoidance lever of the
// Tencent Cloud article, section 4) without swizzling -- and each lane reaches
// all of its fragments at fixed offsets from one base address:
//   K  [D/8 chunk columns][64 keys][16 bytes]
//   V  [D/32 feature blocks][64 keys][32 features]
//
// l is summed from the bf16-rounded P that the PV product consumes (so a row
// dominated by one key normalises exactly), and separately in fp32 for the LSE.
#include "attn_internal.h"
#include "gfx950.h"

namespace attn {

template <int D>
struct FwdTile {
  static constexpr int BC = 64;             // keys per tile
  static constexpr int CH = D / 8;          // 16-byte chunk columns of a K row
  static constexpr int DB = D / 32;         // 32-feature blocks of a V row
  static constexpr int KTILE = CH * BC * 16;
  static constexpr int VTILE = DB * BC * 64;
  static constexpr int SLOT = KTILE + VTILE;
  // 1 KiB pieces per tile: one per K chunk column (64 keys x 16 bytes) and
  // one per (V feature block, 16-key group) (16 keys x 64 bytes).
  static constexpr int NPIECE = CH + DB * (BC / 16);
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p) {
  using T = FwdTile<D>;
  constexpr int NW = 8;
  constexpr int BR = 32 * NW;
  constexpr int BC = T::BC;
  constexpr int NS = 4;          // LDS ring slots
  constexpr int KK = D / 16;     // MFMA steps over the head dimension
  constexpr int DB = D / 32;     // 32-row blocks of O^T
  constexpr int CH = T::CH;
  constexpr int NPW = T::NPIECE / NW;   // tile pieces per wave
  static_assert(T::NPIECE % NW == 0, "tile pieces must split evenly over the waves");

  __shared__ __attribute__((aligned(16))) char smem[NS * T::SLOT];  // [slot][K tile, V tile]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int S = p.S;

  // ---- work unit: (head, query block).  Causal: heaviest query blocks first.
  //      With xcd_heads > 0, consecutive slots of one XCD (workgroup ids are
  //      dealt round-robin over the 8 XCDs) stay on the same heads, so their
  //      K/V re-reads hit that XCD's L2.
  int bh, qi;
  {
    const int u = blockIdx.x;
    if (p.xcd_heads > 0) {
      const int x = u & 7, j = u >> 3, hpx = p.xcd_heads;
      if (CAUSAL) {
        qi = j / hpx;
        bh = x + 8 * (j % hpx);
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

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds row qrow,
  //      features 16*kk + 8*h .. +7 for step kk.
  bf16x8 qf[KK];
  {
    const bool ok = qrow < S;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = *(const u32x4*)(Qh + (size_t)qrow * D + 16 * kk + 8 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (x[e] ^ p.qxor) & p.qand;
      qf[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // keys [0, kend) matter to this workgroup; this wave uses tiles [0, wtiles)
  const int kend = CAUSAL ? min(S, q0 + BR) : S;
  const int ntiles = (kend + BC - 1) / BC;
  const int wend = CAUSAL ? min(S, qw + 32) : S;
  const int wtiles = qw < S ? (wend + BC - 1) / BC : 0;

  // ---- K/V tiles: HBM -> LDS slot directly (rows past S read as zero).
  //      Wave w moves pieces w, w+8, ...: lane l of a K piece carries key l
  //      of one chunk column, lane l of a V piece carries 16 bytes of key l/4
  //      of one feature block, so every piece lands as one 1 KiB run.
  const u32x4 krs = buffer_rsrc(p.k + head, (uint32_t)S * D * 2);
  const u32x4 vrs = buffer_rsrc(p.v + head, (uint32_t)S * D * 2);
  const int kl_off = lane * (2 * D);
  const int vl_off = (lane >> 2) * (2 * D) + (lane & 3) * 16;
  auto fetch = [&](int tile, int slot) {
    const int key0 = tile * BC;
    ATTN_LDS char* base = (ATTN_LDS char*)smem + slot * T::SLOT;
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
      const int i = w + NW * k;   // wave-uniform
      if (i < CH) {
        lds_dma16(base + i * 1024, krs, kl_off, key0 * (2 * D) + i * 16);
      } else {
        const int db = (i - CH) >> 2, rg = (i - CH) & 3;
        lds_dma16(base + T::KTILE + db * (BC * 64) + rg * 1024, vrs, vl_off,
                  (key0 + 16 * rg) * (2 * D) + db * 64);
      }
    }
  };
  // Barriers.  sync_data(k) first waits until this wave's loads of tile k+1
  // have landed (the loads of tile k+2, if requested, may stay in flight), so
  // after it every tile up to k+1 is in LDS for all waves.
  auto sync = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto sync_data = [&](int k) {
    if (k + 2 < ntiles) wait_vmcnt<NPW>();
    else wait_vmcnt<0>();
    sync();
  };

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  float m_run = 0.0f;        // stale row max in log2 units (scores * c); set by tile 0
  float l_b = 0.0f;          // sum of bf16-rounded P (normalises O)
  float l_f = 0.0f;          // sum of fp32 P (for the LSE)
  const float c = p.c;
  const float thresh = p.thresh;   // 2^tau

  // Per-lane LDS byte offsets within a slot; every fragment adds a constant.
  //   K (A operand of S^T): key 32b + l32, chunk column 2kk + h.
  //   V (transposing read, see lds_read_tr16): keys 32b + 16t + 8*half +
  //   tr_key, features 32db + tr_d .. +3.
  const int kbase = h * (BC * 16) + l32 * 16;
  const int vbase = T::KTILE + (4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * 64 +
                    (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  auto slot_ptr = [&](int slot) { return (const ATTN_LDS char*)smem + slot * T::SLOT; };

  // S^T of the tile in slot `slot`: two 32-key blocks
  auto qk = [&](int slot, f32x16 (&s)[2]) {
    const ATTN_LDS char* kb = slot_ptr(slot) + kbase;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16x8 a = lds_read_b128(kb + 2 * kk * (BC * 16) + 32 * b * 16);
        s[b] = mfma32(a, qf[kk], s[b]);
      }
  };
  // O^T += V^T P^T with the tile in slot `slot`
  auto pv = [&](int slot, const uint32_t (&pk)[2][8]) {
    const ATTN_LDS char* vb = slot_ptr(slot) + vbase;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 pw = {pk[b][4 * t], pk[b][4 * t + 1], pk[b][4 * t + 2], pk[b][4 * t + 3]};
        const bf16x8 bp = __builtin_bit_cast(bf16x8, pw);
        const ATTN_LDS char* rb = vb + (32 * b + 16 * t) * 64;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4 x0 = lds_read_tr16(rb + db * (BC * 64));
          const i16x4 x1 = lds_read_tr16(rb + db * (BC * 64) + 8 * 64);
          const u32x4 aw = {__builtin_bit_cast(u32x2, x0)[0], __builtin_bit_cast(u32x2, x0)[1],
                            __builtin_bit_cast(u32x2, x1)[0], __builtin_bit_cast(u32x2, x1)[1]};
          o[db] = mfma32(__builtin_bit_cast(bf16x8, aw), bp, o[db]);
        }
      }
  };
  // The matrix half: S^T of the tile in slot ks and O^T += V^T P^T with the
  // tile in slot vs.  All fragment reads are written first and then
  // interleaved with the products by scheduling groups, so each product finds
  // its operands LA products ahead: LDS latency stays hidden without holding
  // a whole tile in registers.
  auto mphase = [&](int ks, int vs, f32x16 (&s)[2], const uint32_t (&pk)[2][8]) {
    constexpr int NQ = 2 * KK, NP = 4 * DB, NM = NQ + NP, LA = 5;
    const ATTN_LDS char* kb = slot_ptr(ks) + kbase;
    const ATTN_LDS char* vb = slot_ptr(vs) + vbase;
    bf16x8 kf[NQ];
    i16x4 vf[2 * NP];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int b = 0; b < 2; ++b) kf[2 * kk + b] = lds_read_b128(kb + 2 * kk * (BC * 16) + 32 * b * 16);
#pragma unroll
    for (int bt = 0; bt < 4; ++bt)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const ATTN_LDS char* rb = vb + 16 * bt * 64 + db * (BC * 64);
        vf[2 * (DB * bt + db)] = lds_read_tr16(rb);
        vf[2 * (DB * bt + db) + 1] = lds_read_tr16(rb + 8 * 64);
      }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) s[i & 1] = mfma32(kf[i], qf[i >> 1], s[i & 1]);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int bt = i / DB, db = i % DB;
      const u32x4 pw = {pk[bt >> 1][4 * (bt & 1)], pk[bt >> 1][4 * (bt & 1) + 1],
                        pk[bt >> 1][4 * (bt & 1) + 2], pk[bt >> 1][4 * (bt & 1) + 3]};
      const u32x2 a0 = __builtin_bit_cast(u32x2, vf[2 * i]);
      const u32x2 a1 = __builtin_bit_cast(u32x2, vf[2 * i + 1]);
      const u32x4 aw = {a0[0], a0[1], a1[0], a1[1]};
      o[db] = mfma32(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, pw), o[db]);
    }
    MSched<NQ, NM, LA>::apply();
  };
  // keys past the sequence end, and above the causal diagonal, get -inf
  auto mask = [&](int tile, f32x16 (&s)[2]) {
    const int key0 = tile * BC;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
        const bool vis = key < S && (!CAUSAL || key <= qrow);
        if (!vis) s[b][r] = -INFINITY;
      }
  };
  auto needs_mask = [&](int tile) {
    const int key0 = tile * BC;
    return (key0 + BC > S) || (CAUSAL && key0 + BC - 1 > qw);
  };
  auto row_max = [&](const f32x16 (&s)[2]) {
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
    return halfwave_max(mx);
  };
  // pack to bf16 (round to nearest even): the B operand of the PV product
  auto pack = [&](const f32x16 (&e)[2], uint32_t (&pk)[2][8]) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[b][i] = pack_bf16x2(e[b][2 * i], e[b][2 * i + 1]);
  };
  // l_b += the rounded weights of a packed tile (exact products by 1, fp32 sum)
  auto sum_packed = [&](const uint32_t (&pk)[2][8]) {
    float a0 = l_b, a1 = 0.0f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i & 1) a1 = add_bf16x2(pk[b][i], a1);
        else a0 = add_bf16x2(pk[b][i], a0);
      }
    l_b = a0 + a1;
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    l_b *= alpha;
    l_f *= alpha;
  };
  // e = 2^(x - mx) for the kept exponents x; returns this lane's partial sum
  auto expo = [&](const f32x16 (&x)[2], float mx, f32x16 (&e)[2]) {
    float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        e[b][r] = __builtin_amdgcn_exp2f(x[b][r] - mx);
        e[b][r + 1] = __builtin_amdgcn_exp2f(x[b][r + 1] - mx);
        t0 += e[b][r];
        t1 += e[b][r + 1];
      }
    return t0 + t1;
  };
  // Softmax of a later tile against the stale maximum m, with conditional
  // rescaling.  x = s*c - m is kept until the weights e = 2^x have passed the
  // check, so the rare path needs no recomputation of the scores: it moves
  // each row's m up by its largest x (a row whose x never went positive keeps
  // m), scales O and the sums down to match, and redoes the exponentials.
  // Leaves the packed weights in pk and adds them into l_b.
  auto softmax = [&](f32x16 (&s)[2], uint32_t (&pk)[2][8]) {
    const float nm = -m_run;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = __builtin_fmaf(s[b][r], c, nm);
    f32x16 e[2];
    float t = expo(s, 0.0f, e);
    if (wave_any(t > thresh)) {
      const float mx = fmaxf(row_max(s), 0.0f);
      rescale(__builtin_amdgcn_exp2f(-mx));
      m_run += mx;
      t = expo(s, mx, e);
    }
    l_f += t;
    pack(e, pk);
    sum_packed(pk);
  };

  // ---- prologue: tiles 0, 1, 2 requested; wait for 0 and 1; tile 0's
  //      scores and softmax (the row maxima start exact).
  fetch(0, 0);
  if (ntiles > 1) fetch(1, 1);
  if (ntiles > 2) fetch(2, 2);
  sync_data(0);

  uint32_t pk[2][8];
  if (wtiles > 0) {
    f32x16 s[2], e[2];
    qk(0, s);
    if (needs_mask(0)) mask(0, s);
    const float mx = row_max(s);
    m_run = mx == -INFINITY ? 0.0f : mx * c;   // every valid row sees key 0
    const float nm = -m_run;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = __builtin_fmaf(s[b][r], c, nm);
    l_f = expo(s, 0.0f, e);
    pack(e, pk);
    sum_packed(pk);
  }

  // ---- main loop.  Tile j lives in slot j % 4.  Each wave's step j is its
  //      matrix half (which first requests tile j+3 into the slot tile j-1
  //      used), a barrier, its softmax half, and a barrier.  Waves 4..7 start
  //      one barrier late, so their matrix half of step j runs beside the
  //      softmax half of waves 0..3 and vice versa; the matrix half runs at
  //      raised issue priority.  The barrier that ends half-step 2j+2 (after
  //      the softmax half of waves 0..3, after the matrix half of waves 4..7)
  //      is also where every wave waits for its loads of tile j+2, which
  //      waves 0..3 first read right after it.  A wave at its last tile still
  //      runs the score products of the (unused) next slot, so the matrix
  //      half has a single code path.
  const int g = w >> 2;
  if (g == 1) sync();
  for (int j = 0; j < ntiles; ++j) {
    if (j + 3 < ntiles) fetch(j + 3, (j + 3) & (NS - 1));
    f32x16 sn[2];
    if (j < wtiles) {
      __builtin_amdgcn_s_setprio(1);
      mphase((j + 1) & (NS - 1), j & (NS - 1), sn, pk);
      __builtin_amdgcn_s_setprio(0);
    }
    if (g == 0) sync();
    else sync_data(j + 1);
    if (j + 1 < wtiles) {
      if (needs_mask(j + 1)) mask(j + 1, sn);
      softmax(sn, pk);
    }
    if (g == 0) sync_data(j + 1);
    else sync();
  }
  if (g == 0) sync();

  // ---- epilogue: O = O / l (bf16), LSE = ln2 * (m + log2 l)
  const float lb = halfwave_sum(l_b);
  const float lf = halfwave_sum(l_f);
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
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdParams& p0, hipStream_t stream) {
  constexpr int NW = 8;
  FwdParams p = p0;
  p.nqb = (p.S + 32 * NW - 1) / (32 * NW);
  p.xcd_heads = (p.bh % 8 == 0) ? p.bh / 8 : 0;
  p.thresh = exp2f(p.tau);
  const long grid = (long)p.bh * p.nqb;
  if (grid <= 0 || grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<D, CAUSAL>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, stream);
}

hipError_t launch_fwd(const FwdParams& p, int D, bool causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
  if (D == 64) return causal ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
