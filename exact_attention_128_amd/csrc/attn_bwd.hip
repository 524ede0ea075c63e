// attn_bwd.hip -- exact-attention backward for gfx950 (MI355X).
//
// Gradients of sum(dO * O) for O = softmax(scale * Q K^T [causal]) V.  The
// probabilities are never stored: they are recomputed from the forward's LSE
// (the recomputation lever of the Tencent Cloud article "AI Infra 系列 第六章
// GPU 性能工程（二）", section 5).  FA4's backward (same article, section 7)
// reduces dQ with atomics; on MI355X those cost more than recomputing the
// three products dQ needs in a kernel of its own.
//
// Two kernels here, on the caller's stream (dQ is computed by the kernel of
// attn_bwd_dq.hip, which owns query rows, needs no atomics and runs first: it
// also writes the row statistics that the main kernel reads):
//   pre    the row statistics alone, for callers that want them without dQ:
//          per query row of each head, a 16-byte record of -L2_i =
//          -LSE_i * log2(e) and -Delta_i = -sum_d dO_id * O_id (fp32 from the
//          bf16 O, each kept as three bf16 parts; stat_record in gfx950.h),
//          zero for the padding rows past S in the last 64-row block
//   main   dK, dV: one workgroup per (head, 128-key block); each of its 4 waves
//          owns 32 keys, with their K and V rows resident in registers, and
//          walks the query blocks that can see them, 64 queries per step:
//            S   = Q K^T,  dP = dO V^T     (keys on lanes, queries in registers)
//            P   = exp2(S * scale*log2e - L2),  dS = P (dP - Delta)
//          (the dP accumulator starts at -Delta, so dS is a single product;
//          both -L2 and -Delta reach the key lanes through the matrix core:
//          one product of the rows' statistics records against a constant
//          0/1 operand lays each row's value across the tile)
//            dV^T += dO^T P,  dK^T += Q^T dS   (P, dS straight from registers)
//
// Memory pipeline.  Q, dO and the statistics records of a step travel from
// HBM straight into LDS (buffer loads with the LDS destination bit) two steps
// ahead, their load instructions spread over the products of a step; four
// LDS stages, one barrier per step.  The Q/dO tiles are
// stored as [D/8 chunk columns][64 rows][16 bytes] with the chunk columns 64
// bytes apart mod 256, so both fragment reads are free of bank conflicts: the
// 16-byte reads of the score products (32 rows of one chunk column per half
// wave) and the transposing reads of the gradient products (4 rows x 4 chunk
// columns per half wave).
#include <algorithm>
#include <utility>

#include "attn_internal.h"
#include "gfx950.h"

namespace attn {

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ bf16x8 cat_tr(i16x4 a, i16x4 b) {
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  const u32x4 w = {x[0], x[1], y[0], y[1]};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int D>
struct BwdTile {
  static constexpr int BQ = 64;              // queries per step (two 32-query blocks)
  static constexpr int BK = 128;             // keys per workgroup (32 per wave)
  static constexpr int CH = D / 8;           // 16-byte chunk columns of a row
  static constexpr int DB = D / 32;          // 32-feature blocks
  static constexpr int KK = D / 16;          // MFMA steps over the features
  static constexpr int CSTR = BQ * 16 + 64;  // chunk column stride of a Q/dO tile
  static constexpr int QT = CH * CSTR;       // one Q or dO tile
  static constexpr int STAT = 1024;          // 64 rows x 16-byte statistics record
  static constexpr int STAGE = 2 * QT + STAT;
  static constexpr int LDS = 4 * STAGE;      // four stages in flight
  static constexpr int NPC = 2 * CH / 4 + 1; // load instructions per wave and step
  static constexpr int NP = D / 8;           // matrix products per phase of a step
  static constexpr int LA = 6;               // operand reads run this many products ahead
};

// ---------------------------------------------------------------- pre
// Grid-stride over the padded rows: LPR consecutive lanes share a row, and
// the stride is a multiple of LPR, so the lanes of one row always run the
// same iterations (the row's shuffle reduction never reads an idle lane).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(BwdParams p, long rows_pad) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long stride = (long)gridDim.x * 256;
  const int per = p.nblk * 64;
  for (long gid = (long)blockIdx.x * 256 + threadIdx.x; gid < rows_pad * LPR; gid += stride) {
    const long rp = gid / LPR;  // row over [B*H][nblk * 64]
    const int c = (int)(gid % LPR);
    const long bh = rp / per;
    const int r = (int)(rp % per);
    const bool valid = r < p.S;
    const long row = bh * p.S + r;
    float acc = 0.0f;
    if (valid) {
      const u32x4 a = *(const u32x4*)(p.o + row * D + c * 8);
      const u32x4 b = *(const u32x4*)(p.dout + row * D + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(bf16_lo(a[e]), bf16_lo(b[e]), acc);
        acc = __builtin_fmaf(bf16_hi(a[e]), bf16_hi(b[e]), acc);
      }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (c == 0)
      *(u32x4*)(p.stats + (bh * (long)per + r) * 8) =
          stat_record(valid ? -p.lse[row] * kLog2e : 0.0f, valid ? -acc : 0.0f);
  }
}

// ---------------------------------------------------------------- main
//
// One step = queries q0 .. q0+63 of one stage, as blocks A (first 32) and B.
// Its 4*NP matrix products (NP = D/8) form one stream, in four phases:
//   phase 0  S, dP of A      (operand: Q or dO rows, 16-byte reads)
//   phase 1  S, dP of B
//   phase 2  dV^T, dK^T of A (operand: dO^T or Q^T, two transposing reads)
//   phase 3  dV^T, dK^T of B
// The stream is issued in slots, one product per slot, in a fixed order
// (scheduling barriers between slots): each product's LDS operand is read LA
// products ahead of it, so no phase starts by draining the LDS queue, and the
// softmax arithmetic of a block is cut into pairs of elements whose halves
// (exponentials; products and bf16 packing) sit in slots of their own, so the
// exponentials' latency passes while a product issues.  Four LDS stages: the
// loads of step i+2 go to the stage step i-2 read, whose reads all completed
// before the barrier that ended step i-1, so they can be issued anywhere in
// step i.  One load instruction every few slots, not a burst after the
// barrier: with one wave per SIMD a burst holds up the wave's in-order issue,
// its matrix products included, while the CU's load path takes all four
// waves' instructions (spreading them took 2 % off the kernel's time).  The
// single barrier of a step (before the reads of step i+1 start) waits for
// loads issued a step earlier and for no LDS read.
template <int NP, int NPC, int LA>
struct BwdSlots {
  static constexpr bool SPLIT = NP >= 16;  // pair halves in separate slots
  static constexpr int first(int b) { return SPLIT ? (b + 1) * NP + 1 + b : (b + 1) * NP + 1; }
  // slot after whose product half `part` (0: exponentials, 1: products and
  // packing) of element pair k (0..7) of block b is issued
  static constexpr int slot(int b, int k, int part) {
    return SPLIT ? first(b) + 2 * k + part : first(b) + k;
  }
  // the first product that reads pair k of block b (query half k / 4)
  static constexpr int need(int b, int k) { return (2 + b) * NP + (k < 4 ? 0 : NP / 2); }
  // slot after whose product load instruction k (0 .. NPC-1) of step i+2 is
  // issued: spread evenly over the 4 NP - LA slots before the barrier
  static constexpr int load_slot(int k) { return 1 + k * ((4 * NP - LA) / NPC); }
  static constexpr bool valid() {
    if (load_slot(NPC - 1) >= 4 * NP - LA) return false;
    for (int b = 0; b < 2; ++b)
      for (int k = 0; k < 8; ++k)
        if (slot(b, k, 1) >= need(b, k) || slot(b, k, 0) < (b + 1) * NP) return false;
    return true;
  }
};

template <int... M, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, M...>, F&& f) {
  (f(std::integral_constant<int, M>{}), ...);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_main_kernel(BwdParams p) {
  using T = BwdTile<D>;
  constexpr int NW = 4, BQ = T::BQ, BK = T::BK, CH = T::CH, DB = T::DB, KK = T::KK;
  constexpr int CSTR = T::CSTR, QT = T::QT;
  constexpr int NP = T::NP, LA = T::LA, NM = 4 * NP, NX = NM - LA;
  static_assert(2 * KK == NP && 4 * DB == NP, "phase sizes");

  __shared__ __attribute__((aligned(16))) char smem[T::LDS];
  ATTN_LDS char* const lds = (ATTN_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, h = lane >> 5;
  const int g = lane >> 4, ts = lane & 15;  // transposing-read group and slot
  const int S = p.S;

  // ---- work unit: (head, 128-key block).  Ascending key blocks first: under
  //      the causal mask they see the most queries.  With xcd_heads > 0 every
  //      key block of a head runs on one XCD (workgroup ids are dealt
  //      round-robin over the 8 XCDs), so the head's Q/dO re-reads stay in
  //      that XCD's L2.
  int kbi, bh;
  {
    const int u = blockIdx.x;
    if (p.xcd_heads > 0) {
      const int x = u & 7, j = u >> 3;
      kbi = j / p.xcd_heads;
      bh = x + 8 * (j % p.xcd_heads);
    } else {
      kbi = u / p.bh;
      bh = u % p.bh;
    }
  }
  const int k0 = kbi * BK;
  const int kw = k0 + 32 * w;  // first key of this wave
  const int key = kw + l32;    // this lane's key
  const bool kvalid = key < S;
  const size_t head = (size_t)bh * S * D;
  const uint32_t hbytes = (uint32_t)S * D * 2;
  const uint16_t* const stats_h = p.stats + (size_t)bh * p.nblk * 512;  // 1 KiB per 64 rows

  const int qfirst = CAUSAL ? k0 : 0;  // queries before k0 see none of these keys
  const int nsteps = (S - qfirst + BQ - 1) / BQ;

  // ---- step tiles HBM -> LDS stage: Q and dO as [chunk column][64 rows][16 B]
  //      (one 1 KiB load per chunk column, lane l carrying row l; rows past S,
  //      and whole steps past the last, read as zero), then the step's 64
  //      statistics records, which every wave loads (identical bytes) so that
  //      every wave issues the same NPC loads per step, the count the wait at
  //      the step's barrier relies on.
  static_assert(CH % NW == 0 && T::NPC == 2 * CH / NW + 1,
                "chunk columns must split evenly over the waves");
  constexpr int NPC = T::NPC;
  const int row_off = lane * (2 * D);
  // load instruction k of a step's tiles: Q chunk columns (k < CH/NW), dO
  // chunk columns, then the statistics block
  auto fetch_piece = [&](int step, ATTN_LDS char* base, int k) __attribute__((always_inline)) {
    const int q0 = qfirst + step * BQ;
    const uint32_t off = (uint32_t)q0 * (2 * D);
    if (k < 2 * CH / NW) {
      const bool isq = k < CH / NW;
      const int i = w + NW * (isq ? k : k - CH / NW);
      const u32x4 rs = buffer_rsrc_at(isq ? p.q + head : p.dout + head, hbytes, off);
      lds_dma16(base + (isq ? 0 : QT) + i * CSTR, rs, row_off, i * 16);
    } else {
      const u32x4 srs = buffer_rsrc_at(stats_h, (uint32_t)p.nblk * 1024, (uint32_t)(q0 / BQ) * 1024);
      lds_dma16(base + 2 * QT, srs, lane * 16, 0);
    }
  };
  auto fetch = [&](int step, ATTN_LDS char* base) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NPC; ++k) fetch_piece(step, base, k);
  };

  // ---- the first two steps' tiles; K and V rows of this lane's key (B
  //      operands of S and dP: features 16kk + 8h .. +7)
  fetch(0, lds);
  fetch(1, lds + T::STAGE);
  bf16x8 kf[KK], vf[KK];
  {
    const uint16_t* Kr = p.k + head + (size_t)key * D + 8 * h;
    const uint16_t* Vr = p.v + head + (size_t)key * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (kvalid) {
        a = *(const u32x4*)(Kr + 16 * kk);
        b = *(const u32x4*)(Vr + 16 * kk);
      }
      kf[kk] = __builtin_bit_cast(bf16x8, a);
      vf[kk] = __builtin_bit_cast(bf16x8, b);
    }
  }
  wait_all();
  barrier();

  f32x16 dv[DB], dk[DB];  // dV^T, dK^T: lane = key, registers = features
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv[i][r] = 0.0f;
      dk[i][r] = 0.0f;
    }
  const float c = p.c;
  // constant B operands of the statistics products: ones against the record's
  // -L2 parts (elements 0-2) or its -Delta parts (3-5) for the lanes holding
  // k = 0..7, zeros elsewhere (lanes 32-63 hold k = 8..15)
  const bf16x8 ones_l2 = __builtin_bit_cast(
      bf16x8, h == 0 ? u32x4{0x3F803F80u, 0x3F80u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
  const bf16x8 ones_dl = __builtin_bit_cast(
      bf16x8, h == 0 ? u32x4{0u, 0x3F800000u, 0x3F803F80u, 0u} : u32x4{0u, 0u, 0u, 0u});

  // Per-lane LDS offsets (each fragment adds a constant):
  //   qa:  16-byte read of row 32sb + l32, chunk column 2kk + h
  //   tra: transposing read of rows 32sb + 16t + 4(g>>1) + ts/4 (+8), features
  //        32db + 16(g&1) + 4(ts&3) .. +3; rows follow the query order of the
  //        packed P / dS registers
  const int qa_base = h * CSTR + l32 * 16;
  const int tra_base = (2 * (g & 1) + ((ts & 3) >> 1)) * CSTR + (4 * (g >> 1) + (ts >> 2)) * 16 +
                       8 * (ts & 1);

  // LDS operand of product m of a step (phases as above)
  auto operand = [&](const ATTN_LDS char* stg, auto m_t) __attribute__((always_inline)) {
    constexpr int m = decltype(m_t)::value, ph = m / NP, j = m % NP;
    if constexpr (ph < 2) {
      // S (j even: Q) or dP (j odd: dO), features 16(j/2) + 8h .. +7
      return lds_read_b128(stg + qa_base + 512 * ph + (j & 1) * QT + (j >> 1) * 2 * CSTR);
    } else {
      // dV^T (j even: dO^T) or dK^T (j odd: Q^T) of feature block db, query
      // half t of the block
      constexpr int t = j / (2 * DB), db = (j / 2) % DB;
      const ATTN_LDS char* b =
          stg + tra_base + 512 * (ph - 2) + 4 * db * CSTR + 256 * t + ((j & 1) ? 0 : QT);
      return cat_tr(lds_read_tr16(b), lds_read_tr16(b + 128));
    }
  };
  // statistics record of query 32 sb + l32 of a stage (both lane halves read
  // the same record: the A operand of the statistics products, whose k =
  // 8..15 half meets zeros in B but must be finite)
  auto read_rec = [&](const ATTN_LDS char* stg, int sb) {
    return lds_read_b128(stg + 2 * QT + (32 * sb + l32) * 16);
  };
  // Stages rotate over four LDS slots: cur (this step), nxt (step i+1,
  // loaded), fre (read by step i-2, receives step i+2 during this step), and
  // the stage step i-1 read.
  // op holds the operands of the step's first LA products, reca block A's
  // statistics record, on entry; the next step's on exit.
  auto step = [&](auto masked_t, int i, const ATTN_LDS char* cur, const ATTN_LDS char* nxt,
                  ATTN_LDS char* fre, bf16x8 (&op)[LA], bf16x8& reca)
      __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_t)::value;
    constexpr int STAT_B = 2;  // block B's statistics are read after this product
    const int q0 = qfirst + i * BQ;
    bf16x8 o[NM + LA];
    static_for(std::make_integer_sequence<int, LA>{}, [&](auto k) { o[k] = op[k]; });
    f32x16 sacc[2], dacc[2];
    f32x16 nl2[2];  // -L2 of each register's query, in the score layout
    bf16x8 recb;
    uint32_t pk[2][8], dsk[2][8];
    auto product = [&](auto m_t) __attribute__((always_inline)) {
      constexpr int m = decltype(m_t)::value, ph = m / NP, j = m % NP;
      if constexpr (ph < 2) {
        if constexpr ((j & 1) == 0) {
          if constexpr (j == 0) {
            f32x16 z;
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = 0.0f;
            sacc[ph] = mfma32(o[m], kf[0], z);
          } else {
            sacc[ph] = mfma32(o[m], kf[j >> 1], sacc[ph]);
          }
          if constexpr (j == NP - 2) {
            // -L2 tile, late in the phase: its registers live only until
            // the block's softmax has used them
            f32x16 z;
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = 0.0f;
            nl2[ph] = mfma32(ph ? recb : reca, ones_l2, z);
          }
        } else {
          if constexpr (j == 1) {
            f32x16 z;
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = 0.0f;
            dacc[ph] = mfma32(ph ? recb : reca, ones_dl, z);   // -Delta
          }
          dacc[ph] = mfma32(o[m], vf[j >> 1], dacc[ph]);
        }
      } else {
        constexpr int sb = ph - 2, t = j / (2 * DB), db = (j / 2) % DB;
        if constexpr ((j & 1) == 0) {
          const u32x4 pw = {pk[sb][4 * t], pk[sb][4 * t + 1], pk[sb][4 * t + 2], pk[sb][4 * t + 3]};
          dv[db] = mfma32(o[m], __builtin_bit_cast(bf16x8, pw), dv[db]);
        } else {
          const u32x4 sw = {dsk[sb][4 * t], dsk[sb][4 * t + 1], dsk[sb][4 * t + 2],
                            dsk[sb][4 * t + 3]};
          dk[db] = mfma32(o[m], __builtin_bit_cast(bf16x8, sw), dk[db]);
        }
      }
    };
    // softmax pair halves of block b (pair k: elements 2k, 2k+1 = query rows
    // 8(k/2) + 4h + 2(k%2) + {0, 1} of the block): P = exp2(S c - L2) and
    // dS = P (dP - Delta), packed to bf16 in query order.  Lanes of keys past
    // S are left unmasked: a lane's P and dS feed only its own key's dK, dV
    // columns, which are never stored.
    float ex[2][8][2];
    auto half0 = [&](auto b_t, auto k_t) __attribute__((always_inline)) {
      constexpr int b = decltype(b_t)::value, k = decltype(k_t)::value, g4 = k / 2;
      const f32x16& sv = sacc[b];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        constexpr int e0 = 2 * (k % 2);
        float v = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * k + u], c, nl2[b][2 * k + u]));
        if constexpr (MASKED) v = key <= q0 + 32 * b + 8 * g4 + 4 * h + e0 + u ? v : 0.0f;
        ex[b][k][u] = v;
      }
    };
    auto half1 = [&](auto b_t, auto k_t) __attribute__((always_inline)) {
      constexpr int b = decltype(b_t)::value, k = decltype(k_t)::value;
      pk[b][k] = pack_bf16x2(ex[b][k][0], ex[b][k][1]);
      dsk[b][k] = pack_bf16x2(ex[b][k][0] * dacc[b][2 * k], ex[b][k][1] * dacc[b][2 * k + 1]);
    };
    using Sl = BwdSlots<NP, NPC, LA>;
    static_assert(Sl::valid(), "softmax pairs must follow their scores and precede their use");
    static_assert(Sl::slot(1, 7, 1) < NX, "block B's softmax must precede the barrier");
    auto slot = [&](auto m_t) __attribute__((always_inline)) {
      constexpr int m = decltype(m_t)::value;
      product(m_t);
      if constexpr (m < NX) {
        if constexpr (m + LA < NM) o[m + LA] = operand(cur, std::integral_constant<int, m + LA>{});
        if constexpr (m == STAT_B) recb = read_rec(cur, 1);
      } else {
        o[m + LA] = operand(nxt, std::integral_constant<int, m + LA - NM>{});
        if constexpr (m == NX) reca = read_rec(nxt, 0);
      }
      static_for(std::make_integer_sequence<int, NPC>{}, [&](auto k_t) {
        if constexpr (Sl::load_slot(decltype(k_t)::value) == m)
          fetch_piece(i + 2, fre, decltype(k_t)::value);
      });
      static_for(std::make_integer_sequence<int, 2>{}, [&](auto b_t) {
        static_for(std::make_integer_sequence<int, 8>{}, [&](auto k_t) {
          constexpr int b = decltype(b_t)::value, k = decltype(k_t)::value;
          if constexpr (Sl::slot(b, k, 0) == m) half0(b_t, k_t);
          if constexpr (Sl::slot(b, k, 1) == m) half1(b_t, k_t);
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    // ---- before the barrier: products 0 .. NX-1, reads of this stage
    static_for(std::make_integer_sequence<int, NX>{}, slot);
    // ---- step i+1's tiles have landed everywhere (loads retire in order:
    //      only this step's NPC, for step i+2, may still be in flight)
    wait_vmcnt<NPC>();
    barrier();
    __builtin_amdgcn_sched_barrier(0);
    // ---- after the barrier: products NX .. NM-1, reads of step i+1's head
    static_for(std::make_integer_sequence<int, LA>{}, [&](auto k) {
      slot(std::integral_constant<int, NX + decltype(k)::value>{});
    });
    static_for(std::make_integer_sequence<int, LA>{}, [&](auto k) { op[k] = o[NM + k]; });
  };

  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  bf16x8 op[LA];
  static_for(std::make_integer_sequence<int, LA>{}, [&](auto k) { op[k] = operand(lds, k); });
  bf16x8 reca = read_rec(lds, 0);
  // stage rotation: offsets of cur, nxt, fre and the stage step i-1 read
  int sc = 0, sn = T::STAGE, sf = 2 * T::STAGE, sp = 3 * T::STAGE;
  auto rotate = [&]() {
    const int t0 = sc;
    sc = sn;
    sn = sf;
    sf = sp;
    sp = t0;
  };
  int i = 0;
  if constexpr (CAUSAL) {
    // keys k0 .. k0+127 against queries k0 .. k0+127: the only masked steps
    for (; i < 2 && i < nsteps; ++i) {
      step(Yes{}, i, lds + sc, lds + sn, lds + sf, op, reca);
      rotate();
    }
  }
  for (; i < nsteps; ++i) {
    step(No{}, i, lds + sc, lds + sn, lds + sf, op, reca);
    rotate();
  }
  wait_all();  // the loads of the (unused) steps past the end

  // dK = scale * dK^T, dV = dV^T, stored row-major as bf16
  if (kvalid) {
    uint16_t* dkr = p.dk + head + (size_t)key * D;
    uint16_t* dvr = p.dv + head + (size_t)key * D;
    const float sc2 = p.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * h;
        const u32x2 a = {pack_bf16x2(dk[db][4 * g4] * sc2, dk[db][4 * g4 + 1] * sc2),
                         pack_bf16x2(dk[db][4 * g4 + 2] * sc2, dk[db][4 * g4 + 3] * sc2)};
        const u32x2 b = {pack_bf16x2(dv[db][4 * g4], dv[db][4 * g4 + 1]),
                         pack_bf16x2(dv[db][4 * g4 + 2], dv[db][4 * g4 + 3])};
        *(u32x2*)(dkr + d) = a;
        *(u32x2*)(dvr + d) = b;
      }
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p0, unsigned phases, hipStream_t stream) {
  BwdParams p = p0;
  hipError_t e = hipSuccess;
  // the dQ kernel writes the row statistics itself: the separate kernel runs
  // only for callers that ask for them without dQ
  if ((phases & 1u) && !(phases & 4u)) {
    const long rows_pad = (long)p.bh * p.nblk * 64;
    const long threads = rows_pad * (D / 8);
    // at most 1024 workgroups (four per CU), grid-stride beyond: this
    // bandwidth-bound kernel needs no more to fill the chip
    const long grid = std::min((threads + 255) / 256, 1024L);
    void* args[] = {&p, (void*)&rows_pad};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_pre_kernel<D>),
                        dim3((unsigned)grid), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  if (phases & 4u) {
    e = launch_bwd_dq(p, D, CAUSAL, stream);
    if (e != hipSuccess) return e;
  }
  if (phases & 2u) {
    const long nkb = (p.S + BwdTile<D>::BK - 1) / BwdTile<D>::BK;
    const long grid = nkb * p.bh;
    if (grid * 256 > 0xffffffffL) return hipErrorInvalidConfiguration;
    void* args[] = {&p};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_main_kernel<D, CAUSAL>),
                        dim3((unsigned)grid), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return e;
}

hipError_t launch_bwd(const BwdParams& p, int D, bool causal, unsigned phases,
                      hipStream_t stream) {
  if (D == 128)
    return causal ? launch_bwd_t<128, true>(p, phases, stream)
                  : launch_bwd_t<128, false>(p, phases, stream);
  if (D == 64)
    return causal ? launch_bwd_t<64, true>(p, phases, stream)
                  : launch_bwd_t<64, false>(p, phases, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
