// Shared device helpers of libtpmlp: vector types, bf16 conversion, the
// tanh-form GeLU and its derivative, and the LDS chunk swizzle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even on the bit pattern (inputs here are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kPerChunk = 8;  // elements in 16 bytes
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};

// GeLU, tanh form: gelu(x) = x/2 * (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// tanh(u) is evaluated from the identity tanh(u) = 1 - 2 / (exp(2u) + 1) with
// the hardware base-2 exponential and reciprocal (each about 1 ulp); it
// saturates to +-1 correctly when the exponential overflows to inf or
// underflows to 0.
constexpr float kSqrt2OverPi = 0.79788456080286535588f;
constexpr float kGeluCubic = 0.044715f;
constexpr float kTwoLog2e = 2.88539008177792681472f;  // 2 / ln 2

__device__ __forceinline__ float tanh_from_exp(float u) {
  const float e = __builtin_amdgcn_exp2f(u * kTwoLog2e);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

__device__ __forceinline__ float gelu_tanh(float x) {
  float u = kSqrt2OverPi * (x + kGeluCubic * x * x * x);
  return 0.5f * x * (1.0f + tanh_from_exp(u));
}

// d/dx gelu(x) = (1 + t)/2 + x/2 (1 - t^2) sqrt(2/pi) (1 + 3 * 0.044715 x^2).
__device__ __forceinline__ float gelu_tanh_grad(float x) {
  float x2 = x * x;
  float u = kSqrt2OverPi * (x + kGeluCubic * x2 * x);
  float t = tanh_from_exp(u);
  float du = kSqrt2OverPi * (1.0f + 3.0f * kGeluCubic * x2);
  return 0.5f * (1.0f + t) + 0.5f * x * (1.0f - t * t) * du;
}

enum ActKind { kActNone = 0, kActGeluTanh = 1 };

__device__ __forceinline__ float act_apply(int act, float x) {
  return act == kActGeluTanh ? gelu_tanh(x) : x;
}

// LDS tiles hold each row (an M or N index) as 8 chunks of 16 bytes along K.
// Chunk c of row r is stored at position c ^ (r & 7) ^ ((r >> 3) & 7), which
// keeps three access patterns free of bank conflicts: a row written as 8
// chunks, 8 consecutive rows read at one chunk (the MFMA operand reads), and
// 8 rows r = 8g + j (fixed j) written at one chunk (the transposing stores).
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 7); }

}  // namespace tpmlp
