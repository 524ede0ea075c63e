// attn_fwd.hip -- fused exact-attention forward for gfx950 (MI355X).
//
// Computes O = softmax(scale * Q K^T [causal]) V and the natural-log LSE per
// row in one kernel; the S x S scores live only in registers, one K/V tile at
// a time (the tiling + fusion levers of the Tencent Cloud article "AI Infra 系列
// 第六章 GPU 性能工程（二）", section 5; FA4's design in its section 7).
//
// Work decomposition.  A workgroup owns BR = 32 * NW consecutive query rows of
// one (batch, head); each of its NW waves owns 32 of them.  The workgroup walks
// the key/value sequence in tiles of BC = 64 keys staged through LDS (double
// buffered: the global loads of tile j+1 are in flight while tile j is
// consumed).  Per tile and wave:
//
//   S^T = K Q^T     32x32x16 bf16 MFMA; A = K rows from LDS, B = Q held in
//                   registers.  The transposed product puts one query row per
//                   lane (the two wave halves hold different keys of the same
//                   rows), so the row max/sum need only one half-wave swap.
//   mask            only on the tile that crosses the causal diagonal or the
//                   sequence end; tiles wholly above the diagonal are skipped.
//   online softmax  running max m (log2 units) and sum l per row.  The output
//                   is rescaled only when some row's max grew by more than tau
//                   over the stale m in use -- FA4's conditional rescaling
//                   (Tencent Cloud article, section 7).  The stale m cancels
//                   between numerator and denominator, so the result is exact.
//   P = exp2(S c - m) on the hardware exp unit (v_exp_f32, half rate on
//                   gfx950: cheaper than a polynomial on the FMA pipe, so the
//                   pages' software-exp split is not used here).
//   O^T += V^T P^T  32x32x16 bf16 MFMA; B = P straight from registers (bf16),
//                   A = V^T fragments read with the transposing LDS load.
//
// l is summed from the bf16-rounded P that the PV product consumes (so a row
// dominated by one key normalises exactly), and separately in fp32 for the LSE.
#include "attn_internal.h"
#include "gfx950.h"

namespace attn {

template <int D>
struct FwdTile {
  static constexpr int BC = 64;             // keys per tile
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int ROW = D * 2;         // bytes per row
  static constexpr int TILE = BC * ROW;     // bytes per K (or V) tile

  // K tile: row r's chunk c lives at chunk slot c ^ kswz(r).  Sixteen lanes
  // reading one chunk column of sixteen consecutive rows hit 16 distinct
  // 16-byte bank groups.
  __device__ static __forceinline__ int kswz(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
  }
  // V tile: the transposing read fetches 8-byte pieces of 4 consecutive rows x
  // 4 chunks per half wave; rows r and r+4 (the other wave half) are also
  // separated.
  __device__ static __forceinline__ int vswz(int r) {
    return D == 128 ? (((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1))
                    : ((((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1));
  }
};

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p) {
  using T = FwdTile<D>;
  constexpr int BR = 32 * NW;
  constexpr int BC = T::BC;
  constexpr int KK = D / 16;     // MFMA steps over the head dimension
  constexpr int DB = D / 32;     // 32-row blocks of O^T
  constexpr int CH = T::CH;
  constexpr int NT = NW * 64;
  constexpr int LOADS = BC * CH / NT;   // 16-byte chunks per thread per tile
  static_assert((BC * CH) % NT == 0, "tile must split evenly over threads");

  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * T::TILE];  // [buf][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
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
  const uint16_t* __restrict__ Kh = p.k + head;
  const uint16_t* __restrict__ Vh = p.v + head;

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

  // keys [0, kend) matter to this workgroup, keys [0, wend) to this wave
  const int kend = CAUSAL ? min(S, q0 + BR) : S;
  const int wend = CAUSAL ? min(S, qw + 32) : S;
  const int ntiles = (kend + BC - 1) / BC;

  // ---- K/V staging: global -> registers -> LDS (swizzled)
  u32x4 kst[LOADS], vst[LOADS];
  auto gload = [&](int tile) {
    const int key0 = tile * BC;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / CH, c = idx % CH;
      const int key = key0 + row;
      if (key < S) {
        kst[i] = *(const u32x4*)(Kh + (size_t)key * D + c * 8);
        vst[i] = *(const u32x4*)(Vh + (size_t)key * D + c * 8);
      } else {
        kst[i] = u32x4{0u, 0u, 0u, 0u};
        vst[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto lds_store = [&](int buf) {
    char* kb = smem + buf * 2 * T::TILE;
    char* vb = kb + T::TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / CH, c = idx % CH;
      *(u32x4*)(kb + row * T::ROW + ((c ^ T::kswz(row)) << 4)) = kst[i];
      *(u32x4*)(vb + row * T::ROW + ((c ^ T::vswz(row)) << 4)) = vst[i];
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  float m_run = -INFINITY;   // stale row max in log2 units (scores * c)
  float l_b = 0.0f;          // sum of bf16-rounded P (normalises O)
  float l_f = 0.0f;          // sum of fp32 P (for the LSE)
  const float c = p.c;

  // transposing-read geometry for this lane (see lds_read_tr16)
  const int tr_g = lane >> 4, tr_s = lane & 15;
  const int tr_key = 4 * (tr_g >> 1) + (tr_s >> 2);   // + 32*kb + 16*t + 8*half
  const int tr_d = 16 * (tr_g & 1) + 4 * (tr_s & 3);  // + 32*db

  gload(0);
  lds_store(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    if (j + 1 < ntiles) gload(j + 1);
    const int key0 = j * BC;
    if (key0 < wend) {
      const ATTN_LDS char* kb = (const ATTN_LDS char*)(smem + (j & 1) * 2 * T::TILE);
      const ATTN_LDS char* vb = kb + T::TILE;

      // ---- S^T = K Q^T for two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = 0.0f;
        const int row = 32 * b + l32;
        const ATTN_LDS char* rp = kb + row * T::ROW;
        const int sw = T::kswz(row);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 a = lds_read_b128(rp + (((2 * kk + h) ^ sw) << 4));
          s[b] = mfma32(a, qf[kk], s[b]);
        }
      }

      // ---- mask: keys past the sequence end, and above the causal diagonal
      const bool need_mask = (key0 + BC > S) || (CAUSAL && key0 + BC - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool vis = key < S && (!CAUSAL || key <= qrow);
            if (!vis) s[b][r] = -INFINITY;
          }
      }

      // ---- row max and conditional rescale
      float mx = s[0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
      mx = halfwave_max(mx);
      const float m_new = fmaxf(m_run, mx * c);
      if (wave_any(m_new - m_run > p.tau)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
        l_b *= alpha;
        l_f *= alpha;
        m_run = m_new;
      }

      // ---- P = exp2(S c - m), packed to bf16; row sums
      const float nm = -m_run;
      uint32_t pk[2][8];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][2 * i], c, nm));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][2 * i + 1], c, nm));
          pk[b][i] = pack_bf16x2(p0, p1);
          l_b = add_bf16x2(pk[b][i], l_b);
          l_f += p0 + p1;
        }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 pw = {pk[b][4 * t], pk[b][4 * t + 1], pk[b][4 * t + 2], pk[b][4 * t + 3]};
          const bf16x8 bp = __builtin_bit_cast(bf16x8, pw);
          const int kr0 = 32 * b + 16 * t + tr_key;
          const int kr1 = kr0 + 8;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int d = 32 * db + tr_d;
            const i16x4 x0 = lds_read_tr16(vb + kr0 * T::ROW + (((d >> 3) ^ T::vswz(kr0)) << 4) +
                                           (d & 7) * 2);
            const i16x4 x1 = lds_read_tr16(vb + kr1 * T::ROW + (((d >> 3) ^ T::vswz(kr1)) << 4) +
                                           (d & 7) * 2);
            const u32x4 aw = {__builtin_bit_cast(u32x2, x0)[0], __builtin_bit_cast(u32x2, x0)[1],
                              __builtin_bit_cast(u32x2, x1)[0], __builtin_bit_cast(u32x2, x1)[1]};
            o[db] = mfma32(__builtin_bit_cast(bf16x8, aw), bp, o[db]);
          }
        }
    }
    if (j + 1 < ntiles) lds_store((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O / l (bf16), LSE = ln2 * (m + log2 l)
  const float lb = halfwave_sum(l_b);
  const float lf = halfwave_sum(l_f);
  if (qrow < S) {
    const float inv = 1.0f / lb;
    uint16_t* orow = p.o + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * h;
        u32x2 wv = {pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                    pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        *(u32x2*)(orow + d) = wv;
      }
    if (h == 0) p.lse[(size_t)bh * S + qrow] = (m_run + __builtin_amdgcn_logf(lf)) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdParams& p0, hipStream_t stream) {
  constexpr int NW = 4;
  FwdParams p = p0;
  p.nqb = (p.S + 32 * NW - 1) / (32 * NW);
  p.xcd_heads = (p.bh % 8 == 0) ? p.bh / 8 : 0;
  const long grid = (long)p.bh * p.nqb;
  if (grid <= 0 || grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<D, CAUSAL, NW>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, stream);
}

hipError_t launch_fwd(const FwdParams& p, int D, bool causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
  if (D == 64) return causal ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
