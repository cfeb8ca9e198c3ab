// Standalone (unfused) epilogues of the column-parallel layer: the bias and
// GeLU applied to an fp32 product after the GEMM, and GeLU' applied to an
// fp32 input gradient.  The GEMM kernels fuse both into their epilogues; these
// exist as the fusion ablation and for the epilogue's HBM bandwidth.  GeLU
// is elementwise, so it commutes with the column split and each shard applies
// it to its own columns.
//
// Both kernels are HBM-bound: each thread owns 8 consecutive columns of a
// row (two 16-byte fp32 loads, one 16-byte bf16 store per output), rows are
// spread over a grid-stride loop.  Algorithmic bytes per element: 4 (fp32
// input) + 2 x element size (bias_gelu_fwd's two outputs, or gelu_bwd's H
// input and dH output).
#pragma once

#include "common.hpp"

namespace tpmlp {

template <typename T> struct Oct;   // 8 consecutive values of the storage type
template <> struct Oct<bf16_t> {
  u32x4_t w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t x = w[e >> 1];
    return (e & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
  }
  __device__ __forceinline__ void store(bf16_t* p, const float (&v)[8]) const {
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x2_t b = __builtin_convertvector(f32x2_t{v[2 * q], v[2 * q + 1]}, bf16x2_t);   // nearest even
      o[q] = __builtin_bit_cast(uint32_t, b);
    }
    *reinterpret_cast<u32x4_t*>(p) = o;
  }
};
template <> struct Oct<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4_t*>(p);
    b = *reinterpret_cast<const f32x4_t*>(p + 4);
  }
  __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
  __device__ __forceinline__ void store(float* p, const float (&v)[8]) const {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
};

// A = GeLU(Hin + bias), Hs = Hin + bias (Hs optional), N a multiple of 8.
template <typename T>
__global__ void __launch_bounds__(256)
bias_gelu_fwd_kernel(const float* __restrict__ Hin, int64_t ldin, const T* __restrict__ bias, T* __restrict__ A,
                     int64_t lda, T* __restrict__ Hs, int64_t ldh, int rows, int N) {
  const int oct = N / 8;
  const int64_t total = (int64_t)rows * oct;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int r = (int)(i / oct), c = (int)(i - (int64_t)r * oct) * 8;
    const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(Hin + (int64_t)r * ldin + c);
    const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(Hin + (int64_t)r * ldin + c + 4);
    float h[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    if (bias) {
      Oct<T> b;
      b.load(bias + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] += b.get(e);
    }
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = gelu_tanh(h[e]);
    Oct<T> o;
    o.store(A + (int64_t)r * lda + c, a);
    if (Hs) o.store(Hs + (int64_t)r * ldh + c, h);
  }
}

// dH = dA * GeLU'(H), N a multiple of 8.
template <typename T>
__global__ void __launch_bounds__(256)
gelu_bwd_kernel(const float* __restrict__ dA, int64_t ldda, const T* __restrict__ H, int64_t ldh,
                T* __restrict__ dH, int64_t lddh, int rows, int N) {
  const int oct = N / 8;
  const int64_t total = (int64_t)rows * oct;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int r = (int)(i / oct), c = (int)(i - (int64_t)r * oct) * 8;
    const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(dA + (int64_t)r * ldda + c);
    const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(dA + (int64_t)r * ldda + c + 4);
    Oct<T> hv;
    hv.load(H + (int64_t)r * ldh + c);
    const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    float d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = g[e] * gelu_tanh_grad(hv.get(e));
    Oct<T> o;
    o.store(dH + (int64_t)r * lddh + c, d);
  }
}

}  // namespace tpmlp
