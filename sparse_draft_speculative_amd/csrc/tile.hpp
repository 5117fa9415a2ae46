// MFMA / LDS tile helpers shared by the attention and selection kernels
// (gfx950, wave64, v_mfma_f32_16x16x32_bf16).
//
// 16x16x32 bf16 MFMA lane layout (checked on the device): lane l supplies
// A[m = l%16][k = 8*(l/16) + j] and B[k = 8*(l/16) + j][n = l%16], j = 0..7,
// and receives C[m = 4*(l/16) + i][n = l%16], i = 0..3.  Since the product
// sums over k, any permutation of k applied to both operands gives the same
// result; the kernels use that freedom so that each lane's operand is one
// contiguous 16-byte piece of a row.
#pragma once

#include "common.hpp"

namespace stdspec {

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ floatx4_t mfma_bf16(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// ds_read_b64_tr_b16: within each 16-lane group the lanes' 8-byte rows form
// M[16][4]; lane i receives {M[4j + i/4][i%4] : j = 0..3}.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p));
  return __builtin_bit_cast(uint2, t);
}

// LDS tiles of 64 K or V rows, row-major, with the 16-byte chunks of each
// row permuted (XOR swizzle, self-inverse) so that the reads feeding one
// MFMA operand hit distinct banks (measured on the device with the LDS
// bank-conflict counter):
//  * K: chunk c of row r sits at slot c ^ kx(r), kx(r) = (r % 4) * CPR/4 +
//    (r / 4) % (CPR/4).  A K-operand read takes one chunk of 16
//    consecutive rows per 16 lanes.
//  * V: chunk c of row r sits at slot c ^ vx(r), vx(r) = 2 (r % 8) for
//    D = 128 and 2 (r % 4) for D = 64.  A transpose read takes 8 bytes from
//    4 consecutive rows x 2 chunks per 16 lanes.
template <int D>
struct Tile {
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static __device__ __forceinline__ int kx(int row) {
    return (row & 3) * (CPR / 4) + ((row >> 2) & (CPR / 4 - 1));
  }
  static __device__ __forceinline__ int vx(int row) {
    return D == 128 ? (row & 7) << 1 : (row & 3) << 1;
  }
  static __device__ __forceinline__ int slot_k(int row, int chunk) { return chunk ^ kx(row); }
  static __device__ __forceinline__ int slot_v(int row, int chunk) { return chunk ^ vx(row); }
  static __device__ __forceinline__ int off_k(int row, int chunk) {   // elements
    return row * D + (slot_k(row, chunk) << 3);
  }
  static __device__ __forceinline__ int off_v(int row, int chunk) {
    return row * D + (slot_v(row, chunk) << 3);
  }
};

// s_waitcnt immediate: at most n vector-memory operations outstanding
// (gfx9 encoding; expcnt and lgkmcnt left free).
constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

// One direct-to-LDS copy of 16 bytes per lane: lane l's bytes land at
// lds_base + 16 l (lds_base is wave-uniform).  Issued from inline assembly
// so the compiler, which cannot tell which LDS buffer such a copy fills and
// would hold every later LDS read until all copies in flight had landed,
// leaves the ordering to the kernel's explicit vmcnt waits and barriers.
// M0 (the copy's LDS base) is saved and restored around it; one wait state
// separates the M0 write from the copy.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\t"
               "s_mov_b32 m0, %2\n\t"
               "s_nop 0\n\t"
               "global_load_lds_dwordx4 %1, off\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// The same copy with the non-temporal hint, for data a kernel reads exactly
// once (the verify pass's K/V stream): measured faster than the plain copy
// on the 140k-key cache; kernels that re-read their tiles through L2 keep
// the plain form.
__device__ __forceinline__ void dma16_stream(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\t"
               "s_mov_b32 m0, %2\n\t"
               "s_nop 0\n\t"
               "global_load_lds_dwordx4 %1, off nt\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// The 4-byte form: lane l's dword lands at lds_base + 4 l.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\t"
               "s_mov_b32 m0, %2\n\t"
               "s_nop 0\n\t"
               "global_load_lds_dword %1, off\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 cross-row permutes, no LDS round trip.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace stdspec
