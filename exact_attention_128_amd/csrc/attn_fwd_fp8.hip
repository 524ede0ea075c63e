// attn_fwd_fp8.hip -- FP8 (E4M3) exact-attention forward for gfx950 (MI355X).
//
// O = softmax(scale * Q K^T [causal]) V and the natural-log LSE, with Q, K, V
// given as E4M3 codes and one descale factor per tensor (Q = q_descale *
// codes, ...): the precision lever of the Tencent Cloud article "AI Infra 系列
// 第六章 GPU 性能工程（二）", section 5 (lower-precision arithmetic), on the
// gfx950 FP8 matrix core.  Both products run on v_mfma_f32_32x32x64_f8f6f4
// (64-deep contraction, twice the bf16 rate):
//   S^T = K Q^T     A = K rows from LDS (two 16-byte reads: 32 features of the
//                   row per lane), B = Q codes in registers; the products of
//                   two E4M3 values are exact in fp32;
//   O^T += V^T P^T  B = P rounded to E4M3 straight from registers, A = V^T by
//                   the transposing 8-bit LDS read (ds_read_b64_tr_b8: within
//                   each 16 lanes, output lane i takes byte i%8 at the address
//                   of lane 2e + i/8 as its byte e, so lanes pointing at eight
//                   key rows give every output lane one feature of 8 keys).
// The matrix core pairs byte j of lane half h of A with byte j of lane half
// h of B (the same contraction index), so any key or feature order works as
// long as both operands use it: features 64kk + 32h + j for the scores; for
// the PV product the key order of the score accumulators (key 32(j/16) +
// 8((j%16)/4) + 4h + j%4 of a 64-key group), which the V^T reads follow.
//
// Softmax.  As the bf16 kernel (stale maximum, conditional rescale), with the
// weights offset by 2^2 (the first tile's largest weight is exactly 4) and a
// rescale as soon as a lane's step sum passes 2^8: every weight stays at or
// below 256, inside E4M3's finite range (the conversion turns anything from
// 464 up into NaN), and weights down to 2^-10 relative to the offset survive
// as subnormals.  O is normalised by the sum of the E4M3-rounded weights the
// PV product consumes, l^ -- computed by the matrix core itself, one product
// per 64 keys with an all-ones A operand (the matrix core has room here: a
// step's 18 FP8 products take about half the matrix time of the bf16
// kernel's 64) -- and the LSE by the fp32 sum of the unrounded weights.
//
// Work decomposition, LDS rings, load placement and the two-wave ping-pong
// per SIMD are those of the bf16 kernel (attn_fwd.hip); K and V tiles are
// [D/16 chunk columns][64 keys][16 bytes] per 64-key sub-tile, chunk columns
// 1088 bytes apart (a 64-byte skew between columns).
#include "attn_internal.h"
#include "gfx950.h"

namespace attn {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;   // 32 E4M3 codes
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // E4M3 x E4M3 (format selectors 0, 0), no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const ATTN_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS i32x2*)p);
}

__device__ __forceinline__ i32x8 cat2(bf16x8 a, bf16x8 b) {
  const u32x4 x = __builtin_bit_cast(u32x4, a), y = __builtin_bit_cast(u32x4, b);
  const i32x8 r = {(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                   (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
  return r;
}

// four fp32 weights to four E4M3 codes (round to nearest even) in one dword
__device__ __forceinline__ int pack_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Scheduling groups of a matrix half: NQ score products (two 16-byte reads
// each), NP output products (four transposing reads each), NL row-sum
// products (no reads).  The first LA score products' reads were issued
// before the half; after product i come the reads product i + LA needs.
template <int NQ, int NP, int NL, int LA>
struct Fp8Sched {
  static constexpr int NM = NQ + NP + NL;
  static constexpr int need(int i) {
    return i < NQ ? 2 * (i + 1) : (i < NQ + NP ? 2 * NQ + 4 * (i - NQ + 1) : 2 * NQ + 4 * NP);
  }
  template <int I>
  static __device__ __forceinline__ void step() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int more = (I + LA < NM) ? need(I + LA) - need(I + LA - 1) : 0;
    if constexpr (more > 0) __builtin_amdgcn_sched_group_barrier(0x100, more, 0);
  }
  template <int... I>
  static __device__ __forceinline__ void all(std::integer_sequence<int, I...>) {
    (step<I>(), ...);
  }
  static __device__ __forceinline__ void apply() { all(std::make_integer_sequence<int, NM>{}); }
};

}  // namespace

constexpr float kFp8POff = 2.0f;      // log2 offset of the weights (largest first-tile weight 4)
constexpr float kFp8Thresh = 256.0f;  // rescale when a lane's step sum passes 2^8

template <int D>
struct Fp8Tile {
  static constexpr int BC = 64;                 // keys per sub-tile
  static constexpr int CH = D / 16;             // 16-byte chunk columns of a row
  static constexpr int CSTR = BC * 16 + 64;     // chunk column stride
  static constexpr int SUB = CH * CSTR;         // one 64-key sub-tile of K or V
  static constexpr int SLOT = 2 * SUB;          // a step's 128 keys
  static constexpr int NKS = 3;
  static constexpr int NVS = 2;
  static constexpr int LDS = (NKS + NVS) * SLOT;
  static constexpr int PIECE = 2 * CH;          // 1 KiB pieces per step, per tensor
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_kernel(Fp8FwdParams p) {
  using T = Fp8Tile<D>;
  constexpr int NW = 8;
  constexpr int BR = 32 * NW;
  constexpr int BC = T::BC;
  constexpr int KK = D / 64;     // score products per 32-key block
  constexpr int DB = D / 32;     // 32-row blocks of O^T
  constexpr int CH = T::CH;
  constexpr int CSTR = T::CSTR;
  constexpr int PW = T::PIECE / 4;   // pieces per wave of the four that load a tile
  static_assert(T::PIECE % 4 == 0, "pieces must split over 4 waves");

  __shared__ __attribute__((aligned(16))) char smem[T::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int grp = w >> 2;
  const int S = p.S;

  int bh, qi;
  {
    const int u = blockIdx.x;
    if (p.xcd_heads > 0) {
      const int x = u & 7, j = u >> 3;
      if (CAUSAL) {
        // the XCD's heads a group at a time, heaviest block first within it
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

  const int kend = CAUSAL ? min(S, q0 + BR) : S;
  const int nsteps = (kend + 2 * BC - 1) / (2 * BC);
  const int wend = CAUSAL ? min(S, qw + 32) : S;
  const int wsteps = qw < S ? (wend + 2 * BC - 1) / (2 * BC) : 0;

  // ---- K/V tiles HBM -> LDS: piece i = (sub-tile i / CH, chunk column i % CH),
  //      lane l carrying key l of the sub-tile
  const uint32_t hbytes = (uint32_t)S * D;
  const uint8_t* const Kh = p.k + head;
  const uint8_t* const Vh = p.v + head;
  ATTN_LDS char* const kring = (ATTN_LDS char*)smem;
  ATTN_LDS char* const vring = kring + T::NKS * T::SLOT;
  auto fetch = [&](const uint8_t* src, ATTN_LDS char* base, int st) {
    const int key0 = st * 2 * BC;
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int i = (w & 3) + 4 * k;
      const int u = i / CH, cc = i % CH;
      const u32x4 rs = buffer_rsrc_at(src, hbytes, (uint32_t)(key0 + u * BC) * D);
      lds_dma16(base + u * T::SUB + cc * CSTR, rs, lane * D, cc * 16, kPoisonE4M3);
    }
  };
  auto fetch_k = [&](int st) { fetch(Kh, kring + (st % T::NKS) * T::SLOT, st); };
  auto fetch_v = [&](int st) { fetch(Vh, vring + (st % T::NVS) * T::SLOT, st); };
  auto sync = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 o[DB];
  f32x16 lacc;   // l^ of the lane's row in every register
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.0f;
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0
  float m_run = 0.0f;   // stale row max minus the offset, log2 units
  float l_f = 0.0f;     // fp32 sum of the (offset) weights: gives the LSE
  const float c = p.c;

  // per-lane LDS offsets within a sub-tile
  //   K (score A operand): key 32b + l32, features 64kk + 32h .. +31 = chunk
  //   columns 4kk + 2h and 4kk + 2h + 1
  //   V (transposing reads): output lane l = 16g + i holds feature 16(g%2) + i
  //   of a 32-feature block; its address names key
  //   32(r/2) + 16(r%2) + 8(e/4) + 4h + e%4 (read r, e = i/2) at byte 8(i%2)
  const int kbase = 2 * h * CSTR + l32 * 16;
  const int ve = (lane & 15) >> 1;
  const int vbase = ((lane >> 4) & 1) * CSTR + (8 * (ve >> 2) + 4 * h + (ve & 3)) * 16 +
                    8 * (lane & 1);
  auto kslot = [&](int st) { return (const ATTN_LDS char*)kring + (st % T::NKS) * T::SLOT; };
  auto vslot = [&](int st) { return (const ATTN_LDS char*)vring + (st % T::NVS) * T::SLOT; };

  bf16x8 qf2[2 * KK];   // Q codes: features 64kk + 32h .. +15 and +16 .. +31
  // K fragment i of a step: sub-tile u, score step kk, 32-key block b
  auto kfrag = [&](const ATTN_LDS char* kb, int i, bf16x8& lo, bf16x8& hi) {
    const int u = i / (2 * KK), kk = (i % (2 * KK)) >> 1, b = i & 1;
    const ATTN_LDS char* a = kb + u * T::SUB + 4 * kk * CSTR + 32 * b * 16;
    lo = lds_read_b128(a);
    hi = lds_read_b128(a + CSTR);
  };
  auto qk = [&](int st, f32x16 (&s)[4]) {
    const ATTN_LDS char* kb = kslot(st) + kbase;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4 * KK; ++i) {
      bf16x8 lo, hi;
      kfrag(kb, i, lo, hi);
      const int u = i / (2 * KK), kk = (i % (2 * KK)) >> 1, b = i & 1;
      s[2 * u + b] = mfma_fp8(cat2(lo, hi), cat2(qf2[2 * kk], qf2[2 * kk + 1]), s[2 * u + b]);
    }
  };
  constexpr int LA = 3;
  auto kpre_read = [&](int st, bf16x8 (&kp)[2 * LA]) {
    const ATTN_LDS char* kb = kslot(st) + kbase;
#pragma unroll
    for (int i = 0; i < LA; ++i) kfrag(kb, i, kp[2 * i], kp[2 * i + 1]);
  };
  // matrix half: S^T of step ks, O^T += V^T P^T and l^ with the V of step vs
  auto mphase = [&](int ks, int vs, f32x16 (&s)[4], const int (&pk)[2][8],
                    const bf16x8 (&kp)[2 * LA]) {
    constexpr int NQ = 4 * KK, NP = 2 * DB, NL = 2;
    const ATTN_LDS char* kb = kslot(ks) + kbase;
    const ATTN_LDS char* vb = vslot(vs) + vbase;
    bf16x8 kf[2 * NQ];
    i32x2 vf[4 * NP];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i < LA) {
        kf[2 * i] = kp[2 * i];
        kf[2 * i + 1] = kp[2 * i + 1];
      } else {
        kfrag(kb, i, kf[2 * i], kf[2 * i + 1]);
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vf[4 * (DB * g + db) + r] =
              lds_read_tr8(vb + g * T::SUB + 2 * db * CSTR + (r >> 1) * 512 + (r & 1) * 256);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int u = i / (2 * KK), kk = (i % (2 * KK)) >> 1, b = i & 1;
      s[2 * u + b] = mfma_fp8(cat2(kf[2 * i], kf[2 * i + 1]), cat2(qf2[2 * kk], qf2[2 * kk + 1]),
                              s[2 * u + b]);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int g = i / DB, db = i % DB;
      const i32x8 pw = {pk[g][0], pk[g][1], pk[g][2], pk[g][3], pk[g][4], pk[g][5], pk[g][6], pk[g][7]};
      const i32x8 aw = {vf[4 * i][0], vf[4 * i][1], vf[4 * i + 1][0], vf[4 * i + 1][1],
                        vf[4 * i + 2][0], vf[4 * i + 2][1], vf[4 * i + 3][0], vf[4 * i + 3][1]};
      o[db] = mfma_fp8(aw, pw, o[db]);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const i32x8 pw = {pk[g][0], pk[g][1], pk[g][2], pk[g][3], pk[g][4], pk[g][5], pk[g][6], pk[g][7]};
      lacc = mfma_fp8(ones, pw, lacc);
    }
    Fp8Sched<NQ, NP, NL, LA>::apply();
  };
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
  // E4M3 weights of 64-key group g as the PV product's B operand: byte j of
  // the group = register j % 16 of score block 2g + j / 16
  auto pack = [&](const f32x16 (&e)[4], int (&pk)[2][8]) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const f32x16& eb = e[2 * g + (wd >> 2)];
        const int r0 = 4 * (wd & 3);
        pk[g][wd] = pack_e4m3x4(eb[r0], eb[r0 + 1], eb[r0 + 2], eb[r0 + 3]);
      }
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
    l_f *= alpha;
  };
  auto expo = [&](const f32x16 (&x)[4], float mx, f32x16 (&e)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) e[i][r] = __builtin_amdgcn_exp2f(x[i][r] - mx);
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
  // later steps against the stale maximum; a rescale moves each row whose
  // largest (offset) weight passed 2^2 back down to exactly 2^2
  auto softmax = [&](f32x16 (&s)[4], int (&pk)[2][8]) {
    const float nm = -m_run;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = __builtin_fmaf(s[i][r], c, nm);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 e[4];
    float t = expo(s, 0.0f, e);
    if (wave_any(t > kFp8Thresh)) {
      const float mx = fmaxf(row_max(s) - kFp8POff, 0.0f);
      rescale(__builtin_amdgcn_exp2f(-mx));
      m_run += mx;
      t = expo(s, mx, e);
    }
    l_f += t;
    pack(e, pk);
  };

  // ---- prologue (as the bf16 kernel)
  if (grp == 1) fetch_k(0);
  {
    const bool ok = qrow < S;
    const uint8_t* qr = p.q + head + (size_t)(ok ? qrow : S - 1) * D + 32 * h;
    const uint32_t qm = ok ? p.qand : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 x = *(const u32x4*)(qr + 64 * kk + 16 * half);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (x[e] ^ p.qxor) & qm;
        qf2[2 * kk + half] = __builtin_bit_cast(bf16x8, x);
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

  int pk[2][8];
  if (wsteps > 0) {
    f32x16 s[4], e[4];
    qk(0, s);
    if (needs_mask(0)) mask(0, s);
    const float mx = row_max(s);
    m_run = (mx == -INFINITY ? 0.0f : mx * c) - kFp8POff;
    const float nm = -m_run;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = __builtin_fmaf(s[i][r], c, nm);
    l_f = expo(s, 0.0f, e);
    pack(e, pk);
  }

  constexpr int KPW = PW, VPW = PW;
  if (grp == 1) {
    if (nsteps > 2) wait_vmcnt<KPW>();
    else wait_vmcnt<0>();
  } else {
    if (nsteps > 1) wait_vmcnt<VPW>();
    else wait_vmcnt<0>();
  }
  sync();
  bf16x8 kp[2 * LA];
  kpre_read(1, kp);
  if (grp == 1) {
    wait_vmcnt<0>();
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

  // ---- epilogue: O = v_descale * O^T / l^ (bf16), LSE = ln2 * (m + log2 l_f)
  const float lf = halfwave_sum(l_f);
  if (qrow < S) {
    const float inv = p.vscale / lacc[0];
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
    if (h == 0) p.lse[(size_t)bh * S + qrow] = (m_run + __builtin_amdgcn_logf(lf)) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fp8_t(const Fp8FwdParams& p0, hipStream_t stream) {
  constexpr int NW = 8;
  Fp8FwdParams p = p0;
  p.nqb = (p.S + 32 * NW - 1) / (32 * NW);
  p.xcd_heads = (p.bh % 8 == 0) ? p.bh / 8 : 0;
  p.xcd_group = xcd_group(p.xcd_heads, 2L * p.S * D);   // E4M3 K and V of a head
  const long grid = (long)p.bh * p.nqb;
  if (grid <= 0 || grid * NW * 64 > 0xffffffffL) return hipErrorInvalidConfiguration;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_fp8_kernel<D, CAUSAL>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, stream);
}

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int D, bool causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_fp8_t<128, true>(p, stream) : launch_fp8_t<128, false>(p, stream);
  if (D == 64) return causal ? launch_fp8_t<64, true>(p, stream) : launch_fp8_t<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
