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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

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
// Since (1 + tanh(u)) / 2 is the logistic function of 2u, gelu(x) = x * s with
// s = 1 / (1 + exp(-2u)), evaluated with the hardware base-2 exponential and
// reciprocal (each about 1 ulp).  This form has no cancellation for negative
// x, and saturates correctly: exp overflowing to inf gives s = 0, underflow
// to 0 gives s = 1.
constexpr float kGeluZ1 = 2.302208198144325f;     // 2 sqrt(2/pi) / ln 2
constexpr float kGeluZ3 = 0.1029432395800235f;    // the same times 0.044715
constexpr float kGeluD0 = 1.5957691216057308f;    // 2 sqrt(2/pi)
constexpr float kGeluD2 = 0.21406444881780076f;   // the same times 3 * 0.044715

// s = logistic(2u) of the GeLU argument x, and x^2.
__device__ __forceinline__ float gelu_gate(float x, float& x2) {
  x2 = x * x;
  const float z = x * __builtin_fmaf(x2, kGeluZ3, kGeluZ1);  // 2u / ln 2
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z));
}

__device__ __forceinline__ float gelu_tanh(float x) {
  float x2;
  return x * gelu_gate(x, x2);
}

// d/dx gelu(x) = s + x s (1 - s) 2u'(x), u'(x) = sqrt(2/pi) (1 + 3 * 0.044715 x^2).
// x is clamped to +-64 first (the derivative is exactly 0 or 1 in fp32 there),
// so that x^2 stays finite.
__device__ __forceinline__ float gelu_tanh_grad(float x) {
  const float xc = __builtin_amdgcn_fmed3f(x, -64.0f, 64.0f);
  float x2;
  const float s = gelu_gate(xc, x2);
  const float t = xc * __builtin_fmaf(x2, kGeluD2, kGeluD0);  // 2 x u'(x)
  return s * __builtin_fmaf(t, 1.0f - s, 1.0f);
}

// SiLU: silu(g) = g * s, s = 1 / (1 + exp(-g)), with the hardware base-2
// exponential and reciprocal; exp overflowing to inf gives s = 0.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float sigmoidf_fast(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * kLog2e));
}

// d silu / dg = s (1 + g (1 - s)); finite for every finite g.
__device__ __forceinline__ void silu_and_grad(float g, float& silu, float& grad) {
  const float s = sigmoidf_fast(g);
  silu = g * s;
  grad = s * __builtin_fmaf(g, 1.0f - s, 1.0f);
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
