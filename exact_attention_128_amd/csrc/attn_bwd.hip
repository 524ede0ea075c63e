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
// attn_bwd_dq.hip, which owns query rows and needs no atomics):
//   pre    per 64-row block of each head: L2_i = LSE_i * log2(e) and
//          Delta_i = sum_d dO_id * O_id (fp32, from the bf16 O), zero for the
//          padding rows past S
//   main   dK, dV: one workgroup per (head, 128-key block); each of its 4 waves
//          owns 32 keys, with their K and V rows resident in registers, and
//          walks the query blocks that can see them, 64 queries per step:
//            S   = Q K^T,  dP = dO V^T     (keys on lanes, queries in registers)
//            P   = exp2(S * scale*log2e - L2),  dS = P (dP - Delta)
//            dV^T += dO^T P,  dK^T += Q^T dS   (P, dS straight from registers)
//
// Memory pipeline.  Q, dO and the (L2, Delta) block of step i+1 travel from
// HBM straight into LDS (buffer loads with the LDS destination bit) while step
// i computes; two LDS stages, one barrier per step.  The Q/dO tiles are
// stored as [D/8 chunk columns][64 rows][16 bytes] with the chunk columns 64
// bytes apart mod 256, so both fragment reads are free of bank conflicts: the
// 16-byte reads of the score products (32 rows of one chunk column per half
// wave) and the transposing reads of the gradient products (4 rows x 4 chunk
// columns per half wave).
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
  static constexpr int STAT = 1024;          // [L2 x 64][Delta x 64] + landing room
  static constexpr int STAGE = 2 * QT + STAT;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int NPIECE = 2 * CH + 1;  // 1 KiB direct-to-LDS loads per step
};

// ---------------------------------------------------------------- pre
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(BwdParams p, long rows_pad) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long rp = gid / LPR;  // row over [B*H][nblk * 64]
  const int c = (int)(gid % LPR);
  const int per = p.nblk * 64;
  const long bh = rp / per;
  const int r = (int)(rp % per);
  const bool valid = rp < rows_pad && r < p.S;
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
  if (rp < rows_pad && c == 0) {
    float* st = p.stats + bh * (long)per * 2 + (r / 64) * 128 + (r % 64);
    st[0] = valid ? p.lse[row] * kLog2e : 0.0f;
    st[64] = valid ? acc : 0.0f;
  }
}

// ---------------------------------------------------------------- main
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_main_kernel(BwdParams p) {
  using T = BwdTile<D>;
  constexpr int NW = 4, BQ = T::BQ, BK = T::BK, CH = T::CH, DB = T::DB, KK = T::KK;
  constexpr int CSTR = T::CSTR;
  constexpr int PPW = (T::NPIECE + NW - 1) / NW;

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
  const u32x4 qrs = buffer_rsrc(p.q + head, hbytes);
  const u32x4 ors = buffer_rsrc(p.dout + head, hbytes);
  const u32x4 srs = buffer_rsrc(p.stats + (size_t)bh * p.nblk * 128, (uint32_t)p.nblk * 512);

  const int qfirst = CAUSAL ? k0 : 0;  // queries before k0 see none of these keys
  const int nsteps = (S - qfirst + BQ - 1) / BQ;

  // ---- step tiles HBM -> LDS stage: Q and dO as [chunk column][64 rows][16 B]
  //      (one 1 KiB load per chunk column, lane l carrying row l; rows past S,
  //      and whole steps past the last, read as zero), then the step's
  //      (L2, Delta) block, which every wave loads (identical bytes) so that
  //      the issue has no wave-dependent branch.
  static_assert(CH % NW == 0, "chunk columns must split evenly over the waves");
  const int row_off = lane * (2 * D);
  auto fetch = [&](int step, int st) __attribute__((always_inline)) {
    const int q0 = qfirst + step * BQ;
    ATTN_LDS char* base = lds + st * T::STAGE;
#pragma unroll
    for (int k = 0; k < CH / NW; ++k) {
      const int i = w + NW * k;
      lds_dma16(base + i * CSTR, qrs, row_off, q0 * (2 * D) + i * 16);
      lds_dma16(base + T::QT + i * CSTR, ors, row_off, q0 * (2 * D) + i * 16);
    }
    lds_dma16(base + 2 * T::QT, srs, lane * 16, (q0 / BQ) * 512);
  };

  // ---- the first two steps' tiles; K and V rows of this lane's key (B
  //      operands of S and dP: features 16kk + 8h .. +7)
  fetch(0, 0);
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
  fetch(1, 1);

  f32x16 dv[DB], dk[DB];  // dV^T, dK^T: lane = key, registers = features
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv[i][r] = 0.0f;
      dk[i][r] = 0.0f;
    }
  const float c = p.c;

  // Per-lane LDS offsets (each fragment adds a constant):
  //   qa:  16-byte read of row 32sb + l32, chunk column 2kk + h
  //   tra: transposing read of rows 32sb + 16t + 4(g>>1) + ts/4 (+8), features
  //        32db + 16(g&1) + 4(ts&3) .. +3; rows follow the query order of the
  //        packed P / dS registers
  const int qa_base = h * CSTR + l32 * 16;
  const int tra_base = (2 * (g & 1) + ((ts & 3) >> 1)) * CSTR + (4 * (g >> 1) + (ts >> 2)) * 16 +
                       8 * (ts & 1);
  auto stage_ptr = [&](int st) { return (const ATTN_LDS char*)lds + st * T::STAGE; };

  // A operands of S and dP for 32-query block sb: Q then dO, per feature step
  auto read_s = [&](const ATTN_LDS char* stage, int sb, bf16x8 (&f)[2 * KK]) {
    const ATTN_LDS char* qa = stage + qa_base + 512 * sb;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      f[2 * kk] = lds_read_b128(qa + 2 * kk * CSTR);
      f[2 * kk + 1] = lds_read_b128(qa + T::QT + 2 * kk * CSTR);
    }
  };
  // (L2, Delta) of the block's queries 8g4 + 4h .. +3 (broadcast reads)
  auto read_stats = [&](const ATTN_LDS char* stage, int sb, f32x4 (&lv)[4], f32x4 (&dl)[4]) {
    const ATTN_LDS char* sp = stage + 2 * T::QT + 128 * sb + 16 * h;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      lv[g4] = *(const ATTN_LDS f32x4*)(sp + 32 * g4);
      dl[g4] = *(const ATTN_LDS f32x4*)(sp + 256 + 32 * g4);
    }
  };
  // transposed A operands of dV^T (dO) and dK^T (Q): per (t, db) four reads
  auto read_g = [&](const ATTN_LDS char* stage, int sb, i16x4 (&f)[8 * DB]) {
    const ATTN_LDS char* ta = stage + tra_base + 512 * sb;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int o = 4 * db * CSTR + 256 * t, x = 4 * (DB * t + db);
        f[x] = lds_read_tr16(ta + T::QT + o);
        f[x + 1] = lds_read_tr16(ta + T::QT + o + 128);
        f[x + 2] = lds_read_tr16(ta + o);
        f[x + 3] = lds_read_tr16(ta + o + 128);
      }
  };
  // S and dP: C[query][key], lane = key, register r = query 8(r/4) + 4h + r%4
  auto mfma_s = [&](const bf16x8 (&f)[2 * KK], f32x16& s, f32x16& dp) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.0f;
      dp[r] = 0.0f;
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s = mfma32(f[2 * kk], kf[kk], s);
      dp = mfma32(f[2 * kk + 1], vf[kk], dp);
    }
  };
  // P and dS of a 32-query block, packed to bf16 in query order
  auto softmax = [&](auto masked_t, int qb0, const f32x16& s, const f32x16& dp,
                     const f32x4 (&lv)[4], const f32x4 (&dl)[4], uint32_t (&pk)[8],
                     uint32_t (&dsk)[8]) {
    constexpr bool MASKED = decltype(masked_t)::value;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float pr[4], ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g4 + e;
        float v = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lv[g4][e]));
        bool vis = kvalid;
        if constexpr (MASKED) vis = vis && key <= qb0 + 8 * g4 + 4 * h + e;
        v = vis ? v : 0.0f;
        pr[e] = v;
        ds[e] = v * (dp[r] - dl[g4][e]);
      }
      pk[2 * g4] = pack_bf16x2(pr[0], pr[1]);
      pk[2 * g4 + 1] = pack_bf16x2(pr[2], pr[3]);
      dsk[2 * g4] = pack_bf16x2(ds[0], ds[1]);
      dsk[2 * g4 + 1] = pack_bf16x2(ds[2], ds[3]);
    }
  };
  // dV^T += dO^T P, dK^T += Q^T dS
  auto mfma_g = [&](const i16x4 (&f)[8 * DB], const uint32_t (&pk)[8], const uint32_t (&dsk)[8]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pw = {pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]};
      const u32x4 sw4 = {dsk[4 * t], dsk[4 * t + 1], dsk[4 * t + 2], dsk[4 * t + 3]};
      const bf16x8 bp = __builtin_bit_cast(bf16x8, pw);
      const bf16x8 bs = __builtin_bit_cast(bf16x8, sw4);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int x = 4 * (DB * t + db);
        dv[db] = mfma32(cat_tr(f[x], f[x + 1]), bp, dv[db]);
        dk[db] = mfma32(cat_tr(f[x + 2], f[x + 3]), bs, dk[db]);
      }
    }
  };

  // One step: queries qfirst + 64i .. +63 as blocks A (first 32) and B, in
  // four regions that keep the matrix core fed from one wave:
  //   R1  S, dP of A                        reads: S/dP operands of B, stats of A
  //   R2  S, dP of B      + P, dS of A      reads: transposed operands of A, stats of B
  //   R3  dV, dK of A     + P, dS of B      reads: transposed operands of B
  //   --  every LDS read of this stage done, step i+1's loads landed: barrier
  //   R4  dV, dK of B     + loads of step i+2 into this stage, S/dP operands
  //                         of step i+1's block A
  // fa holds block A's S/dP operands on entry and the next step's on exit.
  constexpr int NG = 8 * DB;
  auto step = [&](int i, auto masked_t, bf16x8 (&fa)[2 * KK]) __attribute__((always_inline)) {
    const int st = i & 1;
    const int q0 = qfirst + i * BQ;
    const ATTN_LDS char* stage = stage_ptr(st);
    bf16x8 fb[2 * KK];
    f32x4 lva[4], dla[4], lvb[4], dlb[4];
    i16x4 ga[NG], gb[NG];
    f32x16 sa, dpa, sb, dpb;
    uint32_t pka[8], dsa[8], pkb[8], dsb[8];
    // R1
    read_s(stage, 1, fb);
    read_stats(stage, 0, lva, dla);
    mfma_s(fa, sa, dpa);
    __builtin_amdgcn_sched_barrier(0);
    // R2
    read_g(stage, 0, ga);
    read_stats(stage, 1, lvb, dlb);
    mfma_s(fb, sb, dpb);
    softmax(masked_t, q0, sa, dpa, lva, dla, pka, dsa);
    __builtin_amdgcn_sched_barrier(0);
    // R3
    read_g(stage, 1, gb);
    mfma_g(ga, pka, dsa);
    softmax(masked_t, q0 + 32, sb, dpb, lvb, dlb, pkb, dsb);
    __builtin_amdgcn_sched_barrier(0);
    wait_all();
    barrier();
    // R4
    fetch(i + 2, st);
    read_s(stage_ptr(st ^ 1), 0, fa);
    mfma_g(gb, pkb, dsb);
    __builtin_amdgcn_sched_barrier(0);
  };

  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  bf16x8 fa[2 * KK];
  read_s(stage_ptr(0), 0, fa);
  if constexpr (CAUSAL) {
    // keys k0 .. k0+127 against queries k0 .. k0+127: the only masked steps
    step(0, Yes{}, fa);
    if (nsteps > 1) step(1, Yes{}, fa);
    for (int i = 2; i < nsteps; ++i) step(i, No{}, fa);
  } else {
    for (int i = 0; i < nsteps; ++i) step(i, No{}, fa);
  }
  wait_all();  // the loads of the (unused) steps past the end

  // dK = scale * dK^T, dV = dV^T, stored row-major as bf16
  if (kvalid) {
    uint16_t* dkr = p.dk + head + (size_t)key * D;
    uint16_t* dvr = p.dv + head + (size_t)key * D;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * h;
        const u32x2 a = {pack_bf16x2(dk[db][4 * g4] * sc, dk[db][4 * g4 + 1] * sc),
                         pack_bf16x2(dk[db][4 * g4 + 2] * sc, dk[db][4 * g4 + 3] * sc)};
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
  if (phases & 1u) {
    const long rows_pad = (long)p.bh * p.nblk * 64;
    const long threads = rows_pad * (D / 8);
    const long grid = (threads + 255) / 256;
    void* args[] = {&p, (void*)&rows_pad};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_pre_kernel<D>),
                        dim3((unsigned)grid), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  if (phases & 2u) {
    const long nkb = (p.S + BwdTile<D>::BK - 1) / BwdTile<D>::BK;
    const long grid = nkb * p.bh;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    void* args[] = {&p};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_main_kernel<D, CAUSAL>),
                        dim3((unsigned)grid), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  if (phases & 4u) e = launch_bwd_dq(p, D, CAUSAL, stream);
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
