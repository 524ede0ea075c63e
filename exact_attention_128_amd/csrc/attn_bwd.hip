// attn_bwd.hip -- exact-attention backward for gfx950 (MI355X).
//
// Gradients of sum(dO * O) for O = softmax(scale * Q K^T [causal]) V.  The
// probabilities are never stored: they are recomputed from the forward's LSE
// (the recomputation lever of the Tencent Cloud article "AI Infra 系列 第六章
// GPU 性能工程（二）", section 5); FA4's backward (same article, section 7)
// keeps intermediates on chip and reduces dQ with atomics, as done here.
//
// Three kernels on the caller's stream:
//   pre    Delta_i = sum_d dO_id * O_id (fp32, from the bf16 O), dQacc = 0
//   main   one workgroup per (head, 128-key block); each of its 4 waves owns 32
//          keys with their K and V rows resident in registers, and walks the
//          32-query blocks that can see them:
//            S   = Q K^T,  dP = dO V^T   (keys on lanes, queries in registers)
//            P   = exp2(S * scale*log2e - LSE*log2e),  dS = P (dP - Delta)
//            dV^T += dO^T P,  dK^T += Q^T dS   (P, dS straight from registers)
//            dQacc += dS K   (dS via LDS; fp32 atomics, one add per element
//                             per workgroup and query block)
//   cast   dQ = bf16(scale * dQacc)
#include "attn_internal.h"
#include "gfx950.h"

namespace attn {

namespace {

// LDS swizzle for row-major [rows][D] bf16 tiles that are read both ways: 16
// lanes reading one 16-byte chunk column of 16 consecutive rows (ds_read_b128),
// and the transposing read (4 consecutive rows x 4 chunks per half wave, rows
// r and r+4 in the two halves).  Chunk c of row r is stored at c ^ swz(r).
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1))
                  : ((((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1));
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ bf16x8 cat_tr(i16x4 a, i16x4 b) {
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  const u32x4 w = {x[0], x[1], y[0], y[1]};
  return __builtin_bit_cast(bf16x8, w);
}

}  // namespace

// ---------------------------------------------------------------- pre
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(BwdParams p, long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid / LPR;
  const int c = (int)(gid % LPR);
  float acc = 0.0f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(p.o + row * D + c * 8);
    const u32x4 b = *(const u32x4*)(p.dout + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_fmaf(bf16_lo(a[e]), bf16_lo(b[e]), acc);
      acc = __builtin_fmaf(bf16_hi(a[e]), bf16_hi(b[e]), acc);
    }
    f32x4* z = (f32x4*)(p.dqacc + row * D + c * 8);
    z[0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    z[1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------- cast
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_cast_kernel(BwdParams p, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4* a = (const f32x4*)(p.dqacc + i * 8);
  const f32x4 x = a[0], y = a[1];
  const float s = p.scale;
  const u32x4 w = {pack_bf16x2(x[0] * s, x[1] * s), pack_bf16x2(x[2] * s, x[3] * s),
                   pack_bf16x2(y[0] * s, y[1] * s), pack_bf16x2(y[2] * s, y[3] * s)};
  *(u32x4*)(p.dq + i * 8) = w;
}

// ---------------------------------------------------------------- main
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_main_kernel(BwdParams p) {
  constexpr int NW = 4, BK = 32 * NW, BQ = 32;
  constexpr int KK = D / 16, DB = D / 32, CH = D / 8, ROW = 2 * D, NT = 64 * NW;
  constexpr int DSROW = 2 * BQ;  // bytes per row of the dS^T tile [key][query]

  __shared__ __attribute__((aligned(16))) char sQ[BQ * ROW];
  __shared__ __attribute__((aligned(16))) char sdO[BQ * ROW];
  __shared__ __attribute__((aligned(16))) char sK[BK * ROW];
  __shared__ __attribute__((aligned(16))) char sdS[BK * DSROW];
  __shared__ __attribute__((aligned(16))) float sL[BQ];   // LSE * log2(e) (+inf past S)
  __shared__ __attribute__((aligned(16))) float sDl[BQ];  // Delta (0 past S)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int S = p.S;

  // work unit: key block ascending = most query blocks first under the causal mask
  const int kbi = blockIdx.x / p.bh;
  const int bh = blockIdx.x % p.bh;
  const int k0 = kbi * BK;
  const int kw = k0 + 32 * w;    // first key of this wave
  const int key = kw + l32;      // this lane's key column
  const size_t head = (size_t)bh * S * D;
  const uint16_t* __restrict__ Qh = p.q + head;
  const uint16_t* __restrict__ Kh = p.k + head;
  const uint16_t* __restrict__ Vh = p.v + head;
  const uint16_t* __restrict__ dOh = p.dout + head;
  float* __restrict__ dQh = p.dqacc + head;
  const float* __restrict__ lse = p.lse + (size_t)bh * S;
  const float* __restrict__ dlt = p.delta + (size_t)bh * S;

  // K tile in LDS (B operand of dQ = dS K, read transposed)
  for (int idx = tid; idx < BK * CH; idx += NT) {
    const int row = idx / CH, c = idx % CH, kr = k0 + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (kr < S) x = *(const u32x4*)(Kh + (size_t)kr * D + c * 8);
    *(u32x4*)(sK + row * ROW + ((c ^ swz<D>(row)) << 4)) = x;
  }
  // K and V rows of this lane's key as B operands (features 16*kk + 8*h .. +7)
  bf16x8 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (key < S) {
      a = *(const u32x4*)(Kh + (size_t)key * D + 16 * kk + 8 * h);
      b = *(const u32x4*)(Vh + (size_t)key * D + 16 * kk + 8 * h);
    }
    kf[kk] = __builtin_bit_cast(bf16x8, a);
    vf[kk] = __builtin_bit_cast(bf16x8, b);
  }

  f32x16 dv[DB], dk[DB];  // dV^T, dK^T: lane = key, registers = features
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv[i][r] = 0.0f;
      dk[i][r] = 0.0f;
    }

  const float c = p.c;
  // transposing-read geometry (see lds_read_tr16)
  const int tr_g = lane >> 4, tr_s = lane & 15;
  const int trp_row = 4 * (tr_g >> 1) + (tr_s >> 2);  // P-ordered rows: + 16*t + 8*half
  const int trn_row = 8 * (tr_g >> 1) + (tr_s >> 2);  // natural rows: + 16*ks + 4*half
  const int tr_col = 16 * (tr_g & 1) + 4 * (tr_s & 3);

  const int nqb = (S + BQ - 1) / BQ;
  const int qb0 = CAUSAL ? k0 / BQ : 0;
  const bool wave_has_keys = kw < S;

  for (int qb = qb0; qb < nqb; ++qb) {
    const int q0 = qb * BQ;
    __syncthreads();  // previous block's LDS readers are done
    for (int idx = tid; idx < BQ * CH; idx += NT) {
      const int row = idx / CH, cc = idx % CH, qr = q0 + row;
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (qr < S) {
        x = *(const u32x4*)(Qh + (size_t)qr * D + cc * 8);
        y = *(const u32x4*)(dOh + (size_t)qr * D + cc * 8);
      }
      const int off = row * ROW + ((cc ^ swz<D>(row)) << 4);
      *(u32x4*)(sQ + off) = x;
      *(u32x4*)(sdO + off) = y;
    }
    if (tid < BQ) {
      const int qr = q0 + tid;
      sL[tid] = qr < S ? lse[qr] * kLog2e : INFINITY;
      sDl[tid] = qr < S ? dlt[qr] : 0.0f;
    }
    __syncthreads();

    uint32_t dsk[8];
    const bool active = wave_has_keys && (!CAUSAL || q0 + BQ - 1 >= kw);
    if (active) {
      const ATTN_LDS char* q_l = (const ATTN_LDS char*)sQ;
      const ATTN_LDS char* do_l = (const ATTN_LDS char*)sdO;
      // S = Q K^T and dP = dO V^T: C[query][key], lane = key
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.0f;
        dp[r] = 0.0f;
      }
      const int sw = swz<D>(l32);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int off = l32 * ROW + (((2 * kk + h) ^ sw) << 4);
        s = mfma32(lds_read_b128(q_l + off), kf[kk], s);
        dp = mfma32(lds_read_b128(do_l + off), vf[kk], dp);
      }
      // P and dS; register r holds query 8*(r/4) + 4*h + r%4
      uint32_t pk[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lv = *(const f32x4*)&sL[8 * g + 4 * h];
        const f32x4 dl = *(const f32x4*)&sDl[8 * g + 4 * h];
        float pr[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const int q = q0 + 8 * g + 4 * h + e;
          float v = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lv[e]));
          const bool vis = key < S && q < S && (!CAUSAL || key <= q);
          v = vis ? v : 0.0f;
          pr[e] = v;
          ds[e] = v * (dp[r] - dl[e]);
        }
        pk[2 * g] = pack_bf16x2(pr[0], pr[1]);
        pk[2 * g + 1] = pack_bf16x2(pr[2], pr[3]);
        dsk[2 * g] = pack_bf16x2(ds[0], ds[1]);
        dsk[2 * g + 1] = pack_bf16x2(ds[2], ds[3]);
      }
      // dV^T += dO^T P, dK^T += Q^T dS (A operands read transposed from LDS)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 pw = {pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]};
        const u32x4 sw4 = {dsk[4 * t], dsk[4 * t + 1], dsk[4 * t + 2], dsk[4 * t + 3]};
        const bf16x8 bp = __builtin_bit_cast(bf16x8, pw);
        const bf16x8 bs = __builtin_bit_cast(bf16x8, sw4);
        const int r0 = 16 * t + trp_row, r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = 32 * db + tr_col;
          const int o0 = r0 * ROW + (((d >> 3) ^ swz<D>(r0)) << 4) + (d & 7) * 2;
          const int o1 = r1 * ROW + (((d >> 3) ^ swz<D>(r1)) << 4) + (d & 7) * 2;
          dv[db] = mfma32(cat_tr(lds_read_tr16(do_l + o0), lds_read_tr16(do_l + o1)), bp, dv[db]);
          dk[db] = mfma32(cat_tr(lds_read_tr16(q_l + o0), lds_read_tr16(q_l + o1)), bs, dk[db]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) dsk[i] = 0u;
    }
    // dS^T [key][query] for this wave's 32 keys; 4 consecutive queries per store
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 v2 = {dsk[2 * g], dsk[2 * g + 1]};
      *(u32x2*)(sdS + (32 * w + l32) * DSROW + (8 * g + 4 * h) * 2) = v2;
    }
    __syncthreads();

    // dQ[query][feature] over the block's 128 keys: wave w takes features 32w..32w+31
    if (w < DB && (!CAUSAL || q0 + BQ - 1 >= k0)) {
      const ATTN_LDS char* ds_l = (const ATTN_LDS char*)sdS;
      const ATTN_LDS char* k_l = (const ATTN_LDS char*)sK;
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
      const int d = 32 * w + tr_col;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int r0 = 16 * ks + trn_row, r1 = r0 + 4;
        const bf16x8 a = cat_tr(lds_read_tr16(ds_l + r0 * DSROW + tr_col * 2),
                                lds_read_tr16(ds_l + r1 * DSROW + tr_col * 2));
        const bf16x8 b = cat_tr(
            lds_read_tr16(k_l + r0 * ROW + (((d >> 3) ^ swz<D>(r0)) << 4) + (d & 7) * 2),
            lds_read_tr16(k_l + r1 * ROW + (((d >> 3) ^ swz<D>(r1)) << 4) + (d & 7) * 2));
        acc = mfma32(a, b, acc);
      }
      // C[query][feature]: lane = feature 32w + l32, register r = query 8*(r/4)+4*h+r%4
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (q < S) atomicAdd(dQh + (size_t)q * D + 32 * w + l32, acc[r]);
      }
    }
  }

  // dK = scale * dK^T, dV = dV^T, stored row-major as bf16
  if (key < S) {
    uint16_t* dkr = p.dk + head + (size_t)key * D;
    uint16_t* dvr = p.dv + head + (size_t)key * D;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * h;
        const u32x2 a = {pack_bf16x2(dk[db][4 * g] * sc, dk[db][4 * g + 1] * sc),
                         pack_bf16x2(dk[db][4 * g + 2] * sc, dk[db][4 * g + 3] * sc)};
        const u32x2 b = {pack_bf16x2(dv[db][4 * g], dv[db][4 * g + 1]),
                         pack_bf16x2(dv[db][4 * g + 2], dv[db][4 * g + 3])};
        *(u32x2*)(dkr + d) = a;
        *(u32x2*)(dvr + d) = b;
      }
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p0, unsigned phases, hipStream_t stream) {
  BwdParams p = p0;
  const long rows = (long)p.bh * p.S;
  hipError_t e = hipSuccess;
  if (phases & 1u) {
    const long threads = rows * (D / 8);
    const long grid = (threads + 255) / 256;
    void* args[] = {&p, (void*)&rows};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_pre_kernel<D>),
                        dim3((unsigned)grid), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  if (phases & 2u) {
    const long nkb = (p.S + 127) / 128;
    const long grid = nkb * p.bh;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    void* args[] = {&p};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_main_kernel<D, CAUSAL>),
                        dim3((unsigned)grid), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  if (phases & 4u) {
    const long n8 = rows * D / 8;
    const long grid = (n8 + 255) / 256;
    void* args[] = {&p, (void*)&n8};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dq_cast_kernel<D>),
                        dim3((unsigned)grid), dim3(256), args, 0, stream);
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
