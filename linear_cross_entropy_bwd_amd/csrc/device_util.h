// Device-side helpers: bf16 <-> fp32 conversion and element access traits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace flce {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed pair of bf16 (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return static_cast<bf16_t>(pack_bf16x2(f, 0.0f) & 0xffffu); }

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
};

template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(<N-1>).  Keeps
// register-array indices constant however large the body gets.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr float kLog2e = 1.4426950408889634f;

// exp(x) through the hardware base-2 exponential; exp(-inf) = 0.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

}  // namespace flce
