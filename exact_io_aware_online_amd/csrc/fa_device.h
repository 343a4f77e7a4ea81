// fa_device.h - device-side building blocks shared by the gfx950 kernels.
//
// MFMA operand layouts used throughout (verified on gfx950 by feeding the
// instruction known integer matrices and comparing with a host product):
//   v_mfma_f32_32x32x16_bf16 (lane l, g = l / 32, register i):
//     A[m][k]: m = l % 32, k = 8 g + i   (i = 0..7)
//     B[k][n]: n = l % 32, k = 8 g + i   (i = 0..7)
//     C[m][n]: n = l % 32, m = 8 (i / 4) + 4 g + (i % 4)   (i = 0..15)
//   v_mfma_f32_16x16x32_bf16 (g = l / 16):
//     A[m][k]: m = l % 16, k = 8 g + i;  B[k][n]: n = l % 16, k = 8 g + i
//     C[m][n]: n = l % 16, m = 4 g + i   (i = 0..3)
//   v_mfma_f32_16x16x16_bf16 (g = l / 16):
//     A[m][k]: m = l % 16, k = 4 g + i;  B[k][n]: n = l % 16, k = 4 g + i
//     C[m][n]: n = l % 16, m = 4 g + i
// Only the pairing of A's and B's k index matters for a product, so any
// permutation of k applied to both operands gives the same sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// log2(e): e^x = 2^(x * log2 e). The kernels keep the running maximum in
// base-2 units, t = s * scale * log2(e), and use the hardware 2^x.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(const i16x4& a, const i16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Two floats -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r = {(bf16)lo, (bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// Cross-lane exchange with the lane 32 positions away (the other half of a
// 64-wide wavefront).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// max / sum of x over lanes l and l ^ 32, in both lanes. v_permlane32_swap
// exchanges the upper half of one register with the lower half of another;
// applied to two copies of x it leaves x[l] in one result and x[l ^ 32] in
// the other (which is which does not matter to a symmetric reduction), with
// no LDS round trip.
__device__ __forceinline__ float halves_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// max / sum of x over the four lanes l, l ^ 16, l ^ 32, l ^ 48, in all four:
// v_permlane16_swap exchanges the odd 16-lane rows of one register with the
// even rows of another, which on two copies of x pairs each row with its
// neighbour; the 32-lane swap then pairs the halves.
__device__ __forceinline__ float quarters_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return halves_max(fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])));
}
__device__ __forceinline__ float quarters_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return halves_sum(__builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]));
}

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store_u32x4(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

#define LDS3 __attribute__((address_space(3)))

// Chunk swizzle of a tile row: physical chunk = logical chunk ^ swz(row).
// For rows of 16+ chunks the swizzle depends on row % 16 and spreads the
// 16 consecutive rows a b128 read touches over 16 chunks; pairs of
// consecutive rows (4 rows per transposed read) land on disjoint chunk pairs.
// Rows of 8 chunks (d = 64) are 128 bytes, two per 256-byte bank line, so
// the swizzle follows row / 2 and the row parity supplies the other half.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPR >= 16) {
    return ((row & 7) << 1) | ((row >> 3) & 1);
  } else {
    const int x = (row >> 1) & 7;
    return ((x & 3) << 1) | ((x >> 2) & 1);
  }
}

// Chunk swizzle of the prefill K/V tiles. Their reads take, per LDS cycle,
// one logical chunk of 16 consecutive rows (K, 16-byte reads) or four
// logical chunks of 4 consecutive rows (V, transposing 8-byte reads over 32
// lanes); both touch 64 distinct banks when the two 2-bit digits of
// row % 16 are swapped into the chunk index. Rows of 8 chunks (d = 64) are
// two per 256-byte bank line: there the swizzle follows row / 2 and puts
// the two rows of a line pair into opposite halves of the row.
template <int CPR>
__device__ __forceinline__ int swz_pf(int row) {
  if constexpr (CPR >= 16) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    const int x = (row >> 1) & 7;
    return ((x & 1) << 2) | ((x >> 1) & 3);
  }
}

// One 16-byte direct-to-LDS load per lane: lane l's bytes land at
// lds_addr + 16 l (lds_addr wave-uniform, in M0).
// The base must be wave-uniform; it is passed through readfirstlane so the
// compiler keeps it in SGPRs even where it cannot prove the uniformity.
// An LDS-bound global load reads M0 one wait state after an SALU write of
// M0 at the earliest (the compiler puts an s_nop 0 there in its own code).
// kStream sets the non-temporal hint, for data read once (the decode's
// key/value cache): the caches then treat the lines as streaming, which
// lets a decode move 6-11% more bytes per second on MI355X; data that other
// workgroups read again (the prefill's K/V tiles) must keep the default.
template <bool kStream = false>
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a) |
                     ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32);
  if constexpr (kStream) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"((const void*)(uintptr_t)u), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"((const void*)(uintptr_t)u), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory", "m0");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// s_waitcnt vmcnt(0) issued as a builtin, which the compiler's own wait
// insertion sees: after it, no load into registers issued earlier counts as
// outstanding. Without it the compiler waits for such a load (the Q
// fragment) at its first use inside the tile loop with vmcnt(0) on every
// iteration, which also drains the direct-to-LDS prefetches it cannot see.
// Encoding (gfx9): vmcnt [3:0] and [15:14] = 0, expcnt [6:4] = 7,
// lgkmcnt [11:8] = 15 (no wait on those).
__device__ __forceinline__ void wait_vm_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier after this wavefront's LDS accesses have completed
// (s_waitcnt lgkmcnt(0), issued as a builtin so the compiler's own wait
// insertion sees it). The wait is needed even where every LDS read's result
// is used before the barrier in the source: the compiler may sink a read's
// consumers (MFMAs, which touch no memory) past the barrier while the read
// itself stays ahead of it, and that read could then still be in flight when
// another wavefront, past the barrier, refills the same ring stage.
// Encoding (gfx9): lgkmcnt [11:8] = 0; vmcnt [3:0], [15:14] and expcnt [6:4]
// at their maxima (no wait).
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// An empty statement that reads its operands: every instruction that
// produces them stays ahead of this point in the program (the compiler may
// not sink their computation past it, e.g. into a later block).
__device__ __forceinline__ void materialize(const bf16x8& x) {
  asm volatile("" ::"v"(__builtin_bit_cast(u32x4, x)));
}
__device__ __forceinline__ void materialize(float x) { asm volatile("" ::"v"(x)); }

// x *= s for an accumulator tile held in accumulation registers (AGPRs),
// done in place with read / multiply / write per element. Written as one
// asm statement so that the compiler sees no vector-ALU use of the tile:
// it keeps the tile in AGPRs instead of moving it to VGPRs around a
// rarely taken rescale.
__device__ __forceinline__ void scale_agpr16(f32x16& x, float s) {
  float e0 = x[0], e1 = x[1], e2 = x[2], e3 = x[3], e4 = x[4], e5 = x[5], e6 = x[6], e7 = x[7];
  float e8 = x[8], e9 = x[9], e10 = x[10], e11 = x[11], e12 = x[12], e13 = x[13], e14 = x[14], e15 = x[15];
  float t;
#define FA_SCALE_ONE(i) \
  "v_accvgpr_read_b32 %[t], %[e" #i "]\n\tv_mul_f32 %[t], %[t], %[s]\n\tv_accvgpr_write_b32 %[e" #i "], %[t]\n\t"
  asm volatile(FA_SCALE_ONE(0) FA_SCALE_ONE(1) FA_SCALE_ONE(2) FA_SCALE_ONE(3) FA_SCALE_ONE(4) FA_SCALE_ONE(5)
               FA_SCALE_ONE(6) FA_SCALE_ONE(7) FA_SCALE_ONE(8) FA_SCALE_ONE(9) FA_SCALE_ONE(10) FA_SCALE_ONE(11)
               FA_SCALE_ONE(12) FA_SCALE_ONE(13) FA_SCALE_ONE(14) FA_SCALE_ONE(15)
               : [t] "=&v"(t), [e0] "+a"(e0), [e1] "+a"(e1), [e2] "+a"(e2), [e3] "+a"(e3), [e4] "+a"(e4),
                 [e5] "+a"(e5), [e6] "+a"(e6), [e7] "+a"(e7), [e8] "+a"(e8), [e9] "+a"(e9), [e10] "+a"(e10),
                 [e11] "+a"(e11), [e12] "+a"(e12), [e13] "+a"(e13), [e14] "+a"(e14), [e15] "+a"(e15)
               : [s] "v"(s));
#undef FA_SCALE_ONE
  x = f32x16{e0, e1, e2, e3, e4, e5, e6, e7, e8, e9, e10, e11, e12, e13, e14, e15};
}

// Quiet NaN (bf16 0x7FC0, two per word) over rows [r0, r1) of a bf16 array
// whose row r holds ROWB bytes at base + r * stride; the threads of a
// workgroup share the 16-byte pieces. Packed batches use it to mark every
// output row of a sequence that is longer than the launch covers.
template <int ROWB>
__device__ __forceinline__ void fill_nan_rows(char* base, int64_t stride, int r0, int r1, int tid, int nthreads) {
  constexpr int CPR = ROWB / 16;
  const u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  for (int64_t i = tid; i < (int64_t)(r1 - r0) * CPR; i += nthreads) {
    const int r = r0 + (int)(i / CPR), c = (int)(i % CPR);
    *reinterpret_cast<u32x4*>(base + r * stride + c * 16) = nan4;
  }
}

__device__ __forceinline__ i16x4 ds_read_tr(uint32_t lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 i16x4*)(uintptr_t)lds_addr);
}

}  // namespace fa
