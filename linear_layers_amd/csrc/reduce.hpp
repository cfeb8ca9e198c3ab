// Bandwidth-bound kernels of libtpmlp: the sum of shard partials, the final
// reduction of per-tile column sums, and a zero fill.
#pragma once

#include "common.hpp"

namespace tpmlp {

// out[r, c] = sum_{i < tp} P[i*shard_stride + r*ldp + c], added in ascending i.
// Each thread owns UNROLL 16-byte column groups of a row.  Shards are taken
// in groups of 8 whose loads are all issued before any of their adds, so up
// to 8 * UNROLL loads per thread are in flight; the partials are read once,
// so loads and stores bypass cache residency (non-temporal).  Rows are spread
// over the grid.
template <int UNROLL>
__global__ void __launch_bounds__(256)
partial_sum_kernel(const float* __restrict__ P, int64_t shard_stride, int64_t ldp,
                   float* out, int64_t ldo, int tp, int T, int nvec) {
  const int per_row_blocks = (nvec + 256 * UNROLL - 1) / (256 * UNROLL);
  const int64_t total_blocks = (int64_t)T * per_row_blocks;
  for (int64_t b = blockIdx.x; b < total_blocks; b += gridDim.x) {
    const int r = (int)(b / per_row_blocks);
    const int cb = (int)(b - (int64_t)r * per_row_blocks);
    const float* src = P + (int64_t)r * ldp;
    float* dst = out + (int64_t)r * ldo;
    int cv[UNROLL];
    f32x4_t s[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      cv[u] = (cb * UNROLL + u) * 256 + threadIdx.x;
      s[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int i0 = 0; i0 < tp; i0 += 8) {
      f32x4_t x[8][UNROLL];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
          if (i0 + j < tp && cv[u] < nvec)
            x[j][u] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4_t*>(src + (int64_t)(i0 + j) * shard_stride + 4 * (int64_t)cv[u]));
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
          if (i0 + j < tp && cv[u] < nvec) {
            if (i0 + j == 0) {
              s[u] = x[j][u];
            } else {
              s[u][0] += x[j][u][0];
              s[u][1] += x[j][u][1];
              s[u][2] += x[j][u][2];
              s[u][3] += x[j][u][3];
            }
          }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (cv[u] < nvec) __builtin_nontemporal_store(s[u], reinterpret_cast<f32x4_t*>(dst + 4 * (int64_t)cv[u]));
  }
}

// out[n] = sum_{t < rows} part[t*N + n] in ascending t.  One thread per
// column; eight rows are loaded before they are added, so the loads overlap
// (the sum is latency-bound: a few dozen rows of a few thousand columns).
__global__ void __launch_bounds__(64)
colsum_reduce_kernel(const float* __restrict__ part, int rows, int N, float* __restrict__ out) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= N) return;
  float s = 0.0f;
  int t = 0;
  for (; t + 8 <= rows; t += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(t + u) * N + n];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; t < rows; ++t) s += part[(int64_t)t * N + n];
  out[n] = s;
}

// out[n] = sum_{t < rows} Y[t*ld + n] in fp32: the bias gradient of a linear
// layer from its output gradient.  A block owns 8 chunks of 16 bytes along N
// and 32 row lanes; lane r adds rows r, r+32, ... in order, then the 32 lane
// sums are added in order, so the result does not depend on the launch.
template <typename T>
__global__ void __launch_bounds__(256)
colsum_rows_kernel(const T* __restrict__ Y, int64_t ld, int rows, int N, float* __restrict__ out) {
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int COLS = 8 * EPC;
  __shared__ float part[32][COLS];
  const int cl = threadIdx.x & 7, rl = threadIdx.x >> 3;
  const int c0 = blockIdx.x * COLS + cl * EPC;
  float s[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) s[e] = 0.0f;
  if (c0 < N) {
    for (int r = rl; r < rows; r += 32) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Y + (int64_t)r * ld + c0);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if constexpr (EPC == 8) s[e] += __uint_as_float((e & 1) ? (v[e >> 1] & 0xffff0000u) : (v[e >> 1] << 16));
        else s[e] += __uint_as_float(v[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[rl][cl * EPC + e] = s[e];
  __syncthreads();
  if (threadIdx.x < COLS) {
    const int n = blockIdx.x * COLS + threadIdx.x;
    float t = 0.0f;
    for (int r = 0; r < 32; ++r) t += part[r][threadIdx.x];
    if (n < N) out[n] = t;
  }
}

// Zero rows x cols floats with row stride ld (a kernel, so it is safe inside
// captured graphs, unlike a memset node).
__global__ void __launch_bounds__(256)
fill_zero_kernel(float* __restrict__ p, int rows, int cols, int64_t ld) {
  const int64_t total = (int64_t)rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cols;
    p[r * ld + (i - r * cols)] = 0.0f;
  }
}

}  // namespace tpmlp
