// attn_bwd_dq.hip -- dQ of the exact-attention backward for gfx950 (MI355X).
//
//   dQ_i = scale * sum_j dS_ij K_j,   dS_ij = P_ij (dO_i . V_j - Delta_i),
//   P_ij = exp(scale * Q_i . K_j - LSE_i)
//
// computed per query block, walking the key/value sequence like the forward:
// the probabilities are recomputed from the forward's LSE (the recomputation
// lever of the Tencent Cloud article "AI Infra 系列 第六章 GPU 性能工程（二）",
// section 5), so no softmax rescale is needed.  Each query row's Delta is
// formed here from its O and dO rows, and the row statistics (LSE log2 e,
// -Delta) go to the workspace for the dK/dV kernel, which runs after this one.
// Owning the query rows makes dQ a plain register accumulation: no atomics,
// and the result is deterministic.  (fp32 atomics from the key-block kernel
// would cost more than these three recomputed products on MI355X, whose L2
// completes about 340 G fp32 atomic adds per second.)
//
// Work decomposition, LDS ring and the ping-pong of the two waves of a SIMD
// follow the forward kernel: 8 waves x 32 query rows per workgroup, key tiles
// of 64 in a 4-slot LDS ring filled by direct-to-LDS loads three tiles ahead.
// Each tile step of a wave:
//   matrix half   S^T = K Q^T and dP^T = V dO^T for the NEXT tile (A = K, V
//                 rows from LDS, B = Q, dO rows held in registers), and
//                 dQ^T += K^T dS^T for the CURRENT tile (A = K^T by the
//                 transposing LDS read, B = dS^T straight from registers)
//   softmax half  P = exp2(S c - LSE log2 e), dS = P (dP - Delta), packed bf16
//                 (the dP^T accumulators start at -Delta)
// Query rows sit on lanes, so LSE and Delta are one register each.
//
// LDS slot: K as [D/8 chunk columns][64 keys][16 B] with the chunk columns
// 64 bytes apart mod 256 (16-byte reads: 32 keys of one column per half wave;
// transposing reads: 4 keys x 4 columns per half wave; both conflict-free),
// then V as [D/8 chunk columns][64 keys][16 B].
#include "attn_internal.h"
#include "gfx950.h"

namespace attn {

template <int D>
struct DqTile {
  static constexpr int BC = 64;             // keys per tile
  static constexpr int CH = D / 8;          // 16-byte chunk columns of a row
  static constexpr int DB = D / 32;         // 32-feature blocks
  static constexpr int CSTR = BC * 16 + 64; // K chunk column stride
  static constexpr int KTILE = CH * CSTR;
  static constexpr int VTILE = CH * BC * 16;
  static constexpr int SLOT = KTILE + VTILE;
  static constexpr int NPIECE = 2 * CH;     // 1 KiB loads per tile (one per chunk column)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(BwdParams p) {
  using T = DqTile<D>;
  constexpr int NW = 8;
  constexpr int BR = 32 * NW;
  constexpr int BC = T::BC;
  constexpr int NS = 4;
  constexpr int KK = D / 16;
  constexpr int DB = T::DB;
  constexpr int CH = T::CH;
  constexpr int CSTR = T::CSTR;
  constexpr int NPW = T::NPIECE / NW;
  static_assert(T::NPIECE % NW == 0, "tile pieces must split evenly over the waves");

  __shared__ __attribute__((aligned(16))) char smem[NS * T::SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int g = lane >> 4, ts = lane & 15;
  const int S = p.S;

  // ---- work unit: (head, 256-row query block), heaviest first under the
  //      causal mask; XCD-aware order as in the forward (causal: the XCD's
  //      heads xcd_group at a time, heaviest block first within a group).
  int bh, qi;
  {
    const int u = blockIdx.x;
    if (p.xcd_heads > 0) {
      const int x = u & 7, j = u >> 3;
      if (CAUSAL) {
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
  const int qw = q0 + 32 * w;
  const int qrow = qw + l32;
  const size_t head = (size_t)bh * S * D;

  // ---- this lane's query row: Q' (Q with the sign of the scale folded in,
  //      so that the score multiplier cq is positive and a masked score of
  //      -inf gives P = 0) and dO as B operands (features 16kk + 8h .. +7),
  //      -LSE*log2(e) and -Delta, Delta = sum_d dO_d O_d in fp32 from the
  //      bf16 O (zero past S, which makes dS zero there).  The row statistics
  //      also go to the workspace, one 16-byte record per row
  //      (stat_record), where the dK/dV kernel reads them; rows past S
  //      inside the last 64-row block get zeros there.
  //      The loads are branch-free (a lane past S loads the last row and a
  //      mask zeroes the values), so they issue back to back in the
  //      prologue, behind the first tiles' requests.
  bf16x8 qf[KK], df[KK];
  float nl2 = 0.0f, ndl = 0.0f;
  auto load_rows = [&]() {
    const bool ok = qrow < S;
    const size_t row = (size_t)(ok ? qrow : S - 1);
    const uint16_t* Qr = p.q + head + row * D + 8 * h;
    const uint16_t* Dr = p.dout + head + row * D + 8 * h;
    const uint16_t* Or = p.o + head + row * D + 8 * h;
    const uint32_t qm = ok ? p.qand : 0u;
    const uint32_t rm = ok ? 0xffffffffu : 0u;
    const float lse = p.lse[(size_t)bh * S + row];
    float dsum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 a = *(const u32x4*)(Qr + 16 * kk);
      u32x4 b = *(const u32x4*)(Dr + 16 * kk);
      u32x4 ov = *(const u32x4*)(Or + 16 * kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        b[e] &= rm;
        dsum = __builtin_fmaf(__uint_as_float(b[e] << 16), __uint_as_float(ov[e] << 16), dsum);
        dsum = __builtin_fmaf(__uint_as_float(b[e] & 0xffff0000u),
                              __uint_as_float(ov[e] & 0xffff0000u), dsum);
        a[e] = (a[e] ^ p.qxor) & qm;
      }
      qf[kk] = __builtin_bit_cast(bf16x8, a);
      df[kk] = __builtin_bit_cast(bf16x8, b);
    }
    const float l2 = ok ? lse * kLog2e : 0.0f;
    ndl = -halfwave_sum(dsum);
    nl2 = -l2;
    if (h == 0 && qrow < p.nblk * 64)
      *(u32x4*)(p.stats + ((size_t)bh * p.nblk * 64 + qrow) * 8) = stat_record(nl2, ndl);
  };

  const int kend = CAUSAL ? min(S, q0 + BR) : S;
  const int ntiles = (kend + BC - 1) / BC;
  const int wend = CAUSAL ? min(S, qw + 32) : S;
  const int wtiles = qw < S ? (wend + BC - 1) / BC : 0;

  // ---- K/V tiles HBM -> LDS slot (keys past S read as zero): piece i < CH is
  //      K chunk column i, the rest V chunk columns; lane l carries key l.
  const uint32_t hbytes = (uint32_t)S * D * 2;
  const int row_off = lane * (2 * D);
  auto fetch = [&](int tile, int slot) {
    const uint32_t off = (uint32_t)(tile * BC) * (2 * D);
    const u32x4 krs = buffer_rsrc_at(p.k + head, hbytes, off);
    const u32x4 vrs = buffer_rsrc_at(p.v + head, hbytes, off);
    ATTN_LDS char* base = (ATTN_LDS char*)smem + slot * T::SLOT;
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
      const int i = w + NW * k;  // wave-uniform
      if (i < CH)
        lds_dma16(base + i * CSTR, krs, row_off, i * 16);
      else
        lds_dma16(base + T::KTILE + (i - CH) * (BC * 16), vrs, row_off, (i - CH) * 16);
    }
  };
  auto sync = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 o[DB];  // dQ^T: lane = query row, registers = features
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  f32x16 dinit;  // this lane's -Delta in every register: where dP^T - Delta starts
                 // (set in the prologue)
  const float c = p.cq;

  // Per-lane LDS offsets within a slot (each fragment adds a constant):
  //   16-byte reads: key 32b + l32, chunk column 2kk + h (K, then V)
  //   transposing K reads: keys 32b + 16t + 4(g>>1) + ts/4 (+8), features
  //   32db + 16(g&1) + 4(ts&3) .. +3 -- the key order of the dS^T registers
  const int kbase = h * CSTR + l32 * 16;
  const int vbase = T::KTILE + h * (BC * 16) + l32 * 16;
  const int tbase = (2 * (g & 1) + ((ts & 3) >> 1)) * CSTR + (4 * (g >> 1) + (ts >> 2)) * 16 +
                    8 * (ts & 1);
  auto slot_ptr = [&](int slot) { return (const ATTN_LDS char*)smem + slot * T::SLOT; };

  // S^T and dP^T of the tile in slot `slot` (prologue only)
  auto scores = [&](int slot, f32x16 (&s)[2], f32x16 (&dp)[2]) {
    const ATTN_LDS char* sb = slot_ptr(slot);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[b][r] = 0.0f;
        dp[b][r] = ndl;
      }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[b] = mfma32(lds_read_b128(sb + kbase + 2 * kk * CSTR + 512 * b), qf[kk], s[b]);
        dp[b] = mfma32(lds_read_b128(sb + vbase + 2 * kk * (BC * 16) + 512 * b), df[kk], dp[b]);
      }
  };
  // The matrix half: S^T, dP^T of the tile in slot ns; dQ^T += K^T dS^T with
  // the tile in slot cs.  Fragment reads first, interleaved with the
  // products by scheduling groups (MSched) so each product finds its operands
  // a few products ahead.
  auto mphase = [&](int ns, int cs, f32x16 (&s)[2], f32x16 (&dp)[2],
                    const uint32_t (&pk)[2][8]) {
    constexpr int NQ = 4 * KK, NP = 4 * DB, NM = NQ + NP, LA = 5;
    const ATTN_LDS char* nb = slot_ptr(ns);
    const ATTN_LDS char* tb = slot_ptr(cs) + tbase;
    bf16x8 af[NQ];
    i16x4 tf[2 * NP];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int b = 0; b < 2; ++b) af[2 * kk + b] = lds_read_b128(nb + kbase + 2 * kk * CSTR + 512 * b);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        af[2 * KK + 2 * kk + b] = lds_read_b128(nb + vbase + 2 * kk * (BC * 16) + 512 * b);
#pragma unroll
    for (int bt = 0; bt < 4; ++bt)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const ATTN_LDS char* rb = tb + 4 * db * CSTR + 16 * bt * 16;
        tf[2 * (DB * bt + db)] = lds_read_tr16(rb);
        tf[2 * (DB * bt + db) + 1] = lds_read_tr16(rb + 8 * 16);
      }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < 2 * KK; ++i) s[i & 1] = mfma32(af[i], qf[i >> 1], s[i & 1]);
    // dP^T - Delta: both chains start from the tuple of this lane's -Delta
#pragma unroll
    for (int i = 0; i < 2 * KK; ++i)
      dp[i & 1] = mfma32(af[2 * KK + i], df[i >> 1], i < 2 ? dinit : dp[i & 1]);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int bt = i / DB, db = i % DB;
      const u32x4 pw = {pk[bt >> 1][4 * (bt & 1)], pk[bt >> 1][4 * (bt & 1) + 1],
                        pk[bt >> 1][4 * (bt & 1) + 2], pk[bt >> 1][4 * (bt & 1) + 3]};
      const u32x2 a0 = __builtin_bit_cast(u32x2, tf[2 * i]);
      const u32x2 a1 = __builtin_bit_cast(u32x2, tf[2 * i + 1]);
      const u32x4 aw = {a0[0], a0[1], a1[0], a1[1]};
      o[db] = mfma32(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, pw), o[db]);
    }
    MSched<NQ, NM, LA>::apply();
  };
  auto needs_mask = [&](int tile) {
    const int key0 = tile * BC;
    return (key0 + BC > S) || (CAUSAL && key0 + BC - 1 > qw);
  };
  // Keys past S or above the diagonal get a score of -inf (so P = 0), on the
  // tiles that have any; a separate pass keeps the common softmax branch-free.
  // Element (b, r) holds key key0 + 4h + (32b + 8(r/4) + r%4).
  auto mask = [&](int tile, f32x16 (&s)[2]) {
    const int lim = (CAUSAL ? min(S - 1, qrow) : S - 1) - (tile * BC + 4 * h);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * b + 8 * (r >> 2) + (r & 3) > lim) s[b][r] = -INFINITY;
  };
  // dS^T = P^T (dP^T - Delta), P^T = exp2(S^T c - LSE log2 e), packed to bf16
  // in key order (the B operand of dQ^T); dp already holds dP^T - Delta.  The
  // exponent arguments come first, then all exponentials, then the products:
  // a consumer right behind its v_exp_f32 would stall on the transcendental's
  // latency.
  auto softmax = [&](int tile, f32x16 (&s)[2], f32x16 (&dp)[2], uint32_t (&pk)[2][8]) {
    if (needs_mask(tile)) mask(tile, s);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = __builtin_fmaf(s[b][r], c, nl2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = __builtin_amdgcn_exp2f(s[b][r]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pk[b][i] = pack_bf16x2(s[b][2 * i] * dp[b][2 * i], s[b][2 * i + 1] * dp[b][2 * i + 1]);
  };

  // ---- prologue: tiles 0, 1, 2 requested, then this lane's query row
  //      (above); tile 0's scores and dS.
  fetch(0, 0);
  if (ntiles > 1) fetch(1, 1);
  if (ntiles > 2) fetch(2, 2);
  load_rows();
#pragma unroll
  for (int r = 0; r < 16; ++r) dinit[r] = ndl;
  // A full vmcnt(0) here, visible to the compiler, also retires the Q/dO row
  // loads: the compiler cannot count the direct-to-LDS loads issued as
  // inline assembly, so after a partial wait it would take some row loads as
  // possibly still in flight and re-insert a vmcnt(0) inside every matrix
  // half of the loop, stalling it on the tile loads of the same step.
  wait_vmcnt<0>();
  sync();
  uint32_t pk[2][8];     // dS^T of the tile whose dQ product comes next
  f32x16 sx[2], dpx[2];  // scores of the tile whose softmax comes next
  if (wtiles > 0) {
    scores(0, sx, dpx);
    softmax(0, sx, dpx, pk);
  }

  // ---- main loop: the forward's schedule.  Tile j lives in slot j % 4.
  //      Each wave's step j is its matrix half, a barrier, its softmax half
  //      (which first requests its pieces of tile j+3), and a barrier; waves
  //      4..7 start one barrier late, so on every SIMD one wave's matrix half
  //      (at raised priority) meets the other's softmax half.  Global
  //      barriers 2j and 2j+1 end the matrix halves of step j of waves 0..3
  //      and 4..7; tile m is read between barriers 2m-3 and 2m+1, so tile
  //      j+3 may replace tile j-1 after barrier 2j-1 and must have landed by
  //      barrier 2j+3.  Waves 0..3 request it after barrier 2j and wait for
  //      it before barrier 2j+3 (the end of their next softmax half); waves
  //      4..7 request it after barrier 2j+1 and wait before barrier 2j+3 (the
  //      end of their next matrix half).
  const int grp = w >> 2;
  if (grp == 1) sync();
  for (int j = 0; j < ntiles; ++j) {
    if (j < wtiles) {
      __builtin_amdgcn_s_setprio(1);
      mphase((j + 1) & (NS - 1), j & (NS - 1), sx, dpx, pk);
      __builtin_amdgcn_s_setprio(0);
    }
    if (grp == 1) wait_vmcnt<0>();   // tile j+2, requested in the previous step
    sync();
    if (j + 3 < ntiles) fetch(j + 3, (j + 3) & (NS - 1));
    if (j + 1 < wtiles) softmax(j + 1, sx, dpx, pk);
    if (grp == 0) {   // tile j+2, requested in the previous step
      if (j + 3 < ntiles) wait_vmcnt<NPW>();
      else wait_vmcnt<0>();
    }
    sync();
  }
  if (grp == 0) sync();

  // ---- epilogue: dQ = scale * dQ^T, row-major bf16
  if (qrow < S) {
    const float sc = p.scale;
    uint16_t* dqr = p.dq + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * h;
        const u32x2 wv = {pack_bf16x2(o[db][4 * g4] * sc, o[db][4 * g4 + 1] * sc),
                          pack_bf16x2(o[db][4 * g4 + 2] * sc, o[db][4 * g4 + 3] * sc)};
        *(u32x2*)(dqr + d) = wv;
      }
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_dq_t(const BwdParams& p0, hipStream_t stream) {
  constexpr int NW = 8;
  BwdParams p = p0;
  p.nqb = (p.S + 32 * NW - 1) / (32 * NW);
  p.xcd_group = xcd_group(p.xcd_heads, 4L * p.S * D);   // bf16 K and V of a head
  const long grid = (long)p.bh * p.nqb;
  if (grid <= 0 || grid * NW * 64 > 0xffffffffL) return hipErrorInvalidConfiguration;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D, CAUSAL>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, stream);
}

hipError_t launch_bwd_dq(const BwdParams& p, int D, bool causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_dq_t<128, true>(p, stream) : launch_dq_t<128, false>(p, stream);
  if (D == 64) return causal ? launch_dq_t<64, true>(p, stream) : launch_dq_t<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
