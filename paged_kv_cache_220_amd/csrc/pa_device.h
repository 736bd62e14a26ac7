// Device helpers for the PagedAttention decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace pa {

// Storage-type tags (match pa_dtype_t).
enum : int { kF32 = 0, kBF16 = 1, kE5M2 = 2, kE4M3 = 3, kI4 = 4 };

template <int T> struct Storage;
template <> struct Storage<kF32> { using type = float; };
template <> struct Storage<kBF16> { using type = uint16_t; };
template <> struct Storage<kE5M2> { using type = uint8_t; };
template <> struct Storage<kE4M3> { using type = uint8_t; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// OCP E5M2 is the upper byte of an IEEE binary16 with the same value, so the
// conversion is exact for every code (subnormals, infinities and NaNs included).
__device__ __forceinline__ float e5m2_to_f32(uint32_t byte) {
  const uint16_t h = static_cast<uint16_t>((byte & 0xFFu) << 8);
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

template <int T> __device__ __forceinline__ float to_f32(typename Storage<T>::type x);
template <> __device__ __forceinline__ float to_f32<kF32>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<kBF16>(uint16_t x) { return bf16_bits_to_f32(x); }
template <> __device__ __forceinline__ float to_f32<kE5M2>(uint8_t x) { return e5m2_to_f32(x); }
// OCP E4M3 (bias 7, no infinities, S.1111.111 = NaN): gfx950's fp8 convert reads this format.
template <> __device__ __forceinline__ float to_f32<kE4M3>(uint8_t x) { return __builtin_amdgcn_cvt_f32_fp8(x, 0); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

template <int T> __device__ __forceinline__ void store_out(void* out, int64_t idx, float x);
template <> __device__ __forceinline__ void store_out<kF32>(void* out, int64_t idx, float x) {
  static_cast<float*>(out)[idx] = x;
}
template <> __device__ __forceinline__ void store_out<kBF16>(void* out, int64_t idx, float x) {
  static_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(x);
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): indices
// known at compile time (register rings and LDS stages never indexed at run time).
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

}  // namespace pa
