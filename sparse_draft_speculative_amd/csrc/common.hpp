// Device helpers shared by the gfx950 kernels of the StD hot path.
//
// wave64 throughout.  bf16 values travel as raw 16-bit patterns (uint16_t)
// and are widened exactly to fp32 by a shift; fp32 -> bf16 rounds to nearest
// even through the compiler's __bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stdspec {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
// Native 16-byte vector for register staging (HIP's uint4 class is copied
// through memory, which keeps arrays of it out of registers).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b));
}

// Pack two fp32 values into one dword of two bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {   // bf16 bit patterns
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float x) {
    p[i] = static_cast<uint16_t>(f32_to_bf16_bits(x));
  }
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// log2(e): softmax runs in the base-2 domain, exp(x) = exp2(x * log2 e).
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace stdspec
