// gfx950.h -- small device helpers for the CDNA4 (gfx950) attention kernels:
// vector types for the bf16 matrix-core operands, LDS address-space casts,
// bf16 packing, and the half-wave exchange used by the row reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace attn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 matrix FMA, fp32 accumulate.  Lane layout (checked on gfx950):
//   A (32 x 16):  lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//   B (16 x 32):  lane l holds B[8 * (l / 32) + e][l % 32]
//   C (32 x 32):  lane l, register r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 values to two bf16 (round to nearest even), packed into 32 bits.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// The backward's row-statistics record, 16 bytes per query row: a and b
// (-LSE*log2(e) and -Delta) each as the sum of three bf16 parts, hi + mid +
// lo, then two zero parts: [a0 a1 a2 b0 b1 b2 0 0].  Each part is the
// round-to-nearest-even bf16 of what the earlier parts leave (the
// differences are exact in fp32), so the three reproduce the value to about
// 2^-26 relative.  The dK/dV kernel feeds the record to the matrix core as
// an A operand against constant 0/1 B operands, which adds the parts back in
// fp32 and lays one row's value across every key lane of the output tile.
__device__ __forceinline__ u32x4 stat_record(float a, float b) {
  auto bf = [](float x) { return __uint_as_float(pack_bf16x2(x, 0.0f) << 16); };
  const float a0 = bf(a), a1 = bf(a - a0), a2 = (a - a0) - a1;
  const float b0 = bf(b), b1 = bf(b - b0), b2 = (b - b0) - b1;
  return u32x4{pack_bf16x2(a0, a1), pack_bf16x2(a2, b0), pack_bf16x2(b1, b2), 0u};
}

// Value held by the lane in the other half of the wave (lane ^ 32), combined.
__device__ __forceinline__ float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// 16-byte LDS read (ds_read_b128).
__device__ __forceinline__ bf16x8 lds_read_b128(const ATTN_LDS char* p) {
  return *(const ATTN_LDS bf16x8*)p;
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// output lane 16g+i, element e (e = 0..3) receives the 16-bit word at
// (address supplied by lane 16g + 4e + i/4) + 2*(i % 4) bytes.  With the
// source lanes pointing at four consecutive rows of a row-major bf16 matrix
// (lanes 4e..4e+3 of the group covering 16 consecutive columns of row e),
// every output lane gets one column's four row values.
__device__ __forceinline__ i16x4 lds_read_tr16(const ATTN_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)p);
}

// One direct-to-LDS load: each lane's 16 bytes at buffer offset voff + soff
// land at dst + 16 * lane.  Issued as inline assembly on purpose: the kernel
// orders these loads against its LDS reads itself (a vmcnt wait plus a
// barrier per tile), and a compiler that sees the LDS write adds conservative
// waits for it in front of unrelated LDS reads.  The memory clobber keeps LDS
// accesses from moving across it.
// (Nothing else in these kernels uses m0, so clobbering it is safe.)
//
// LDS race check (debug build, compiled with ATTN_LDS_POISON=1 into
// libattn_lds_poison.so): before each such load the lane writes a NaN pattern
// over the 16 bytes the load will land, and waits for that write.  A wave
// that reads a piece before the load's wait and barrier -- a missing wait, or
// a refill that overtakes the piece's last reader -- then reads NaN instead of
// an older tile, and the NaN reaches the outputs; so does a load that leaves
// its bytes unwritten (rows past the end must land as zeros).
#ifndef ATTN_LDS_POISON
#define ATTN_LDS_POISON 0
#endif
constexpr uint32_t kPoisonBf16 = 0x7FC07FC0u;   // bf16 NaN pairs, also an fp32 NaN
constexpr uint32_t kPoisonE4M3 = 0x7F7F7F7Fu;   // E4M3 NaN bytes
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(ATTN_LDS char* dst, u32x4 rsrc, int voff, int soff,
                                          uint32_t poison = kPoisonBf16) {
  if constexpr (ATTN_LDS_POISON != 0) {
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    ATTN_LDS uint32_t* const d = (ATTN_LDS uint32_t*)(dst + 16 * lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = poison;   // four 4-byte stores: one register
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the pattern has landed
  } else {
    (void)poison;
  }
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// vmcnt(0) and lgkmcnt(0): every memory access this wave issued has completed.
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Raw buffer descriptor (gfx9 layout) over nbytes at base, in SGPRs.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const u32x4 r = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) & 0xffffu,
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)nbytes), 0x00020000u};
  return r;
}

// Descriptor over bytes [off, nbytes) of the array at base (empty when off >=
// nbytes): a load through it starts at the array's byte off.  The kernels
// put a tile's first row at off and only a within-row byte offset in the
// load's scalar offset, so the descriptor's size bounds every lane's row by
// the array's true end (rows past it read as zero) whether or not the
// hardware counts the scalar offset in its range check.
__device__ __forceinline__ u32x4 buffer_rsrc_at(const void* base, uint32_t nbytes, uint32_t off) {
  return buffer_rsrc((const char*)base + off, off < nbytes ? nbytes - off : 0u);
}

// Scheduling groups for a matrix half: NQ score products (one 16-byte LDS read
// each) then NM - NQ output products (two 8-byte transposing reads each).
// The reads of the first LA products go first (none when PRE: the caller
// read those operands before the half began); after product i come the reads
// that product i + LA needs.
template <int NQ, int NM, int LA, bool PRE = false>
struct MSched {
  static constexpr int need(int i) { return i < NQ ? i + 1 : NQ + 2 * (i - NQ + 1); }
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
  static __device__ __forceinline__ void apply() {
    if constexpr (!PRE) __builtin_amdgcn_sched_group_barrier(0x100, need(LA - 1), 0);
    all(std::make_integer_sequence<int, NM>{});
  }
};

}  // namespace attn
