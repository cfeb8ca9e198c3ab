// Storage-order kernels of the gated MLP (SwiGLU) block.
//
// The joined first-layer shard [W_gate_i | W_up_i] is kept interleaved in
// groups of 8 columns: packed column 16q + r is gate column 8q + r (r < 8) or
// up column 8q + r - 8 (r >= 8) of shard i's F/tp columns (wangyu.me,
// 大语言模型并行策略（三）：张量并行, 多层感知机（MLP）中的张量并行: the two
// weights may be joined along their columns so that one product yields both).
// Both kernels move whole 8-element chunks; one thread per chunk.
#pragma once

#include "common.hpp"

namespace tpmlp {

template <typename T>
struct Chunk8 {  // 8 elements: one 16-byte vector for bf16, two for fp32
  static constexpr int kVec = sizeof(T) * 8 / 16;
  u32x4_t v[kVec];
  __device__ __forceinline__ void load(const T* p) {
#pragma unroll
    for (int k = 0; k < kVec; ++k) v[k] = reinterpret_cast<const u32x4_t*>(p)[k];
  }
  __device__ __forceinline__ void store(T* p) const {
#pragma unroll
    for (int k = 0; k < kVec; ++k) reinterpret_cast<u32x4_t*>(p)[k] = v[k];
  }
};

// W_gu [rows, 2 Fs] (contiguous) from columns [c0, c0 + Fs) of W_gate and W_up.
template <typename T>
__global__ void __launch_bounds__(256) swiglu_pack_kernel(const T* __restrict__ Wg, int64_t ldg,
                                                          const T* __restrict__ Wu, int64_t ldu, int64_t c0,
                                                          int rows, int Fs, T* __restrict__ Wgu) {
  const int chunks = Fs / 4;  // packed chunks per row: 2 Fs / 8
  const int64_t total = (int64_t)rows * chunks;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
    const int r = (int)(t / chunks), pc = (int)(t % chunks);
    const int q = pc >> 1;
    const T* src = (pc & 1) ? Wu + (int64_t)r * ldu : Wg + (int64_t)r * ldg;
    Chunk8<T> c;
    c.load(src + c0 + 8 * q);
    c.store(Wgu + (int64_t)r * (2 * (int64_t)Fs) + 8 * pc);
  }
}

// Columns [c0, c0 + Fs) of dW_gate and dW_up from the packed dW_gu [rows, 2 Fs].
__global__ void __launch_bounds__(256) swiglu_unpack_kernel(const float* __restrict__ dWgu, int rows, int Fs,
                                                            int64_t c0, float* __restrict__ dWg, int64_t ldg,
                                                            float* __restrict__ dWu, int64_t ldu) {
  const int chunks = Fs / 4;
  const int64_t total = (int64_t)rows * chunks;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
    const int r = (int)(t / chunks), pc = (int)(t % chunks);
    const int q = pc >> 1;
    float* dst = (pc & 1) ? dWu + (int64_t)r * ldu : dWg + (int64_t)r * ldg;
    Chunk8<float> c;
    c.load(dWgu + (int64_t)r * (2 * (int64_t)Fs) + 8 * pc);
    c.store(dst + c0 + 8 * q);
  }
}

}  // namespace tpmlp
