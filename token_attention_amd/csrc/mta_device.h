// Device-side helpers for gfx950: MFMA operand traits and wave reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace mta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16x16 MFMA tiles. For every element type the operand layout is the same:
//   A (16 x K): lane l holds row (l & 15), k = (l >> 4) * KPL + [0, KPL)
//   B (K x 16): lane l holds col (l & 15), k = (l >> 4) * KPL + [0, KPL)
//   D (16 x 16, fp32): lane l holds col (l & 15), rows 4 * (l >> 4) + [0, 4)
// so an operand is always read from a row-major array as "row (l & 15), KPL
// consecutive elements starting at column (l >> 4) * KPL".
template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  static constexpr int K = 32;
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  static __device__ __forceinline__ frag load(const __bf16* p) {
    return *reinterpret_cast<const frag*>(p);
  }
  static __device__ __forceinline__ frag zero() { return frag{}; }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<_Float16> {
  static constexpr int K = 32;
  static constexpr int KPL = 8;
  typedef f16x8 frag;
  static __device__ __forceinline__ frag load(const _Float16* p) {
    return *reinterpret_cast<const frag*>(p);
  }
  static __device__ __forceinline__ frag zero() { return frag{}; }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int K = 4;
  static constexpr int KPL = 1;
  typedef float frag;
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ frag zero() { return 0.0f; }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Reductions over the 16 lanes that share (l >> 4): the columns of one D-layout row.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 4));
  x = fmaxf(x, __shfl_xor(x, 8));
  return x;
}

__device__ __forceinline__ float row16_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ T to_elem(float x) {
  return static_cast<T>(x);
}

}  // namespace mta
