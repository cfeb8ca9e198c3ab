// Kernels of the sequence-parallel (SP) region around the tensor-parallel
// block: LayerNorm over one GPU's rows of the sequence, and the
// reduce-scatter end of the block fused with Dropout and the residual add.
//
// io.zouht.com/197.html, 2.2.2 与序列并行（Sequence Parallel）结合: Dropout is
// elementwise and LayerNorm normalises each hidden state by its own mean and
// (biased) variance, so both split along the sequence; 2.3 代价: the forward
// all-reduce becomes an all-gather before the block and a reduce-scatter
// after it.  sunjinbo.space/document/parallelism.html, SP · 序列并行: the
// residual add belongs to the same sequence-split region.
//
// Dropout draws its bits from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): element (r, c) of
// the [T, h] tensor (r the global row) takes word e % 4, e = r*h + c, of the
// generator at counter (n mod 2^32, n >> 32, 0, 0), n = e / 4, keyed by the
// 64-bit seed; it is kept iff that word >= a threshold floor(p * 2^32).
#pragma once

#include "common.hpp"

namespace tpmlp {

// ------------------------------------------------------------ Philox4x32 --
constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;  // round multipliers
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;  // key increments

__device__ __forceinline__ u32x4_t philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint32_t hi0 = __umulhi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
    const uint32_t hi1 = __umulhi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return u32x4_t{c0, c1, c2, c3};
}

// Keep flags of the 8 elements e0 .. e0 + 7 (e0 a multiple of 8).
__device__ __forceinline__ uint32_t keep8(uint64_t e0, uint64_t seed, uint32_t thr) {
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint64_t n = (e0 >> 2) + q;
    const u32x4_t w = philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), 0u, 0u, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
    for (int j = 0; j < 4; ++j) bits |= (w[j] >= thr ? 1u : 0u) << (4 * q + j);
  }
  return bits;
}

__device__ __forceinline__ void unpack8(const u32x4_t v, float (&x)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(v[k] << 16);
    x[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4_t pack8(const float (&x)[8]) {
  u32x4_t v;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2_t p = __builtin_convertvector(f32x2_t{x[2 * k], x[2 * k + 1]}, bf16x2_t);  // RNE
    v[k] = __builtin_bit_cast(uint32_t, p);
  }
  return v;
}

// Sum over the 256 threads of a workgroup, in a fixed order (deterministic).
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) v += __shfl_xor(v, x);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red may still be read from a previous call
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

constexpr int kLnMaxChunks = 8;  // 8-element chunks per thread: rows up to 256 * 8 * 8 = 16384 wide

// ------------------------------------------------------------- LayerNorm --
// One workgroup of 256 threads per row (measured faster than one wave per
// row, which leaves too few waves per CU to hide the load latency).  The row
// stays in registers: mean, then the biased variance around it, then
// Y = gamma * (x - mean) * rstd + beta.
constexpr int kLnThreads = 256;  // threads per row

__global__ void __launch_bounds__(256) layernorm_fwd_kernel(const bf16_t* __restrict__ X, int64_t ldx, int rows, int h,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta, float eps,
                                                            bf16_t* __restrict__ Y, int64_t ldy,
                                                            float* __restrict__ mean, float* __restrict__ rstd) {
  __shared__ float red[4];
  const int tr = threadIdx.x;
  const int64_t r = blockIdx.x;
  (void)rows;
  const int chunks = h >> 3;
  float x[kLnMaxChunks][8];
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kLnMaxChunks; ++k) {
    const int c = tr + kLnThreads * k;
    if (c < chunks) {
      unpack8(*reinterpret_cast<const u32x4_t*>(X + r * ldx + 8 * c), x[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += x[k][e];
    }
  }
  const float mu = block_sum256(s, red) / (float)h;
  float q = 0.0f;
#pragma unroll
  for (int k = 0; k < kLnMaxChunks; ++k) {
    if (tr + kLnThreads * k < chunks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = x[k][e] - mu;
        q += d * d;
      }
    }
  }
  const float var = block_sum256(q, red) / (float)h;
  const float rs = rsqrtf(var + eps);
#pragma unroll
  for (int k = 0; k < kLnMaxChunks; ++k) {
    const int c = tr + kLnThreads * k;
    if (c < chunks) {
      const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(gamma + 8 * c);
      const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(gamma + 8 * c + 4);
      const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(beta + 8 * c);
      const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(beta + 8 * c + 4);
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = (x[k][e] - mu) * rs * g0[e] + b0[e];
        y[4 + e] = (x[k][4 + e] - mu) * rs * g1[e] + b1[e];
      }
      *reinterpret_cast<u32x4_t*>(Y + r * ldy + 8 * c) = pack8(y);
    }
  }
  if (tr == 0) {
    mean[r] = mu;
    rstd[r] = rs;
  }
}

// dX = rstd * (g - mean(g) - xhat * mean(g * xhat)) (+ dRes), g = dY * gamma,
// xhat = (x - mean) * rstd; one workgroup per row as in the forward.
__global__ void __launch_bounds__(256) layernorm_bwd_kernel(const bf16_t* __restrict__ X, int64_t ldx, int rows, int h,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ mean,
                                                            const float* __restrict__ rstd,
                                                            const float* __restrict__ dY, int64_t lddy,
                                                            const bf16_t* __restrict__ dRes, int64_t ldr,
                                                            float* __restrict__ dX, int64_t lddx) {
  __shared__ float red[4];
  const int tr = threadIdx.x;
  const int64_t r = blockIdx.x;
  (void)rows;
  const int chunks = h >> 3;
  const float mu = mean[r], rs = rstd[r];
  float xh[kLnMaxChunks][8], g[kLnMaxChunks][8];
  float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
  for (int k = 0; k < kLnMaxChunks; ++k) {
    const int c = tr + kLnThreads * k;
    if (c < chunks) {
      unpack8(*reinterpret_cast<const u32x4_t*>(X + r * ldx + 8 * c), xh[k]);
      const f32x4_t d0 = *reinterpret_cast<const f32x4_t*>(dY + r * lddy + 8 * c);
      const f32x4_t d1 = *reinterpret_cast<const f32x4_t*>(dY + r * lddy + 8 * c + 4);
      const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(gamma + 8 * c);
      const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(gamma + 8 * c + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[k][e] = d0[e] * g0[e];
        g[k][4 + e] = d1[e] * g1[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xh[k][e] = (xh[k][e] - mu) * rs;
        s1 += g[k][e];
        s2 += g[k][e] * xh[k][e];
      }
    }
  }
  const float m1 = block_sum256(s1, red) / (float)h;
  const float m2 = block_sum256(s2, red) / (float)h;
#pragma unroll
  for (int k = 0; k < kLnMaxChunks; ++k) {
    const int c = tr + kLnThreads * k;
    if (c < chunks) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = rs * (g[k][e] - m1 - xh[k][e] * m2);
      if (dRes) {
        float d[8];
        unpack8(*reinterpret_cast<const u32x4_t*>(dRes + r * ldr + 8 * c), d);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += d[e];
      }
      *reinterpret_cast<f32x4_t*>(dX + r * lddx + 8 * c) = f32x4_t{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4_t*>(dX + r * lddx + 8 * c + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
    }
  }
}

// dgamma[c] = sum_r dY[r,c] * xhat[r,c], dbeta[c] = sum_r dY[r,c].  A
// workgroup owns 16 columns (4 chunks of 4) and 64 row lanes; lane l adds rows
// l, l + 64, ... in order, then the 64 lane sums are added in order.
// Workgroups are dealt to the 8 XCDs in turn, and a 128-byte line of X spans
// four column groups (of dY, two): column group g therefore goes to the
// workgroup on XCD g / q (q = full groups per XCD), so the groups that share
// lines run on one XCD and read them through its L2 once.
__global__ void __launch_bounds__(256) layernorm_param_grad_kernel(const bf16_t* __restrict__ X, int64_t ldx,
                                                                   int rows, int h, const float* __restrict__ mean,
                                                                   const float* __restrict__ rstd,
                                                                   const float* __restrict__ dY, int64_t lddy,
                                                                   float* __restrict__ dgamma,
                                                                   float* __restrict__ dbeta) {
  __shared__ float pg[64][16], pb[64][16];
  const int cl = threadIdx.x & 3, rl = threadIdx.x >> 2;
  const int q = (int)(gridDim.x >> 3), b = (int)blockIdx.x;
  const int grp = b < 8 * q ? (b & 7) * q + (b >> 3) : b;
  const int c0 = grp * 16 + 4 * cl;
  float sg[4] = {0.f, 0.f, 0.f, 0.f}, sb[4] = {0.f, 0.f, 0.f, 0.f};
  if (c0 < h) {
#pragma unroll 4
    for (int r = rl; r < rows; r += 64) {
      const f32x4_t d = *reinterpret_cast<const f32x4_t*>(dY + (int64_t)r * lddy + c0);
      const u32x2_t xw = *reinterpret_cast<const u32x2_t*>(X + (int64_t)r * ldx + c0);
      const float xv[4] = {__uint_as_float(xw[0] << 16), __uint_as_float(xw[0] & 0xffff0000u),
                           __uint_as_float(xw[1] << 16), __uint_as_float(xw[1] & 0xffff0000u)};
      const float mu = mean[r], rs = rstd[r];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sg[e] += d[e] * ((xv[e] - mu) * rs);
        sb[e] += d[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pg[rl][4 * cl + e] = sg[e];
    pb[rl][4 * cl + e] = sb[e];
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    const int col = threadIdx.x & 15;
    const bool beta_half = threadIdx.x >= 16;
    float t = 0.0f;
    for (int l = 0; l < 64; ++l) t += beta_half ? pb[l][col] : pg[l][col];
    const int n = grp * 16 + col;
    if (n < h) {
      if (beta_half) {
        if (dbeta) dbeta[n] = t;
      } else if (dgamma) {
        dgamma[n] = t;
      }
    }
  }
}

// ------------------------------------------------- reduce-scatter + dropout --
// out[r] = residual[r] + Dropout(sum_s partials[s][r]) for rows r of this GPU's
// block (global row row0 + r); shards are added in ascending order in fp32,
// loaded eight at a time before their adds.  One thread per 8-element chunk.
__global__ void __launch_bounds__(256) sp_sum_dropout_residual_kernel(
    const float* __restrict__ P, int64_t shard_stride, int64_t ldp, int tp, int rows, int h,
    const bf16_t* __restrict__ res, int64_t ldr, uint32_t thr, float scale, uint64_t seed, int64_t row0,
    bf16_t* __restrict__ out, int64_t ldo) {
  const uint32_t cpr = (uint32_t)h >> 3;
  const uint32_t total = (uint32_t)rows * cpr;  // < 2^31, checked on the host
  for (uint32_t t = blockIdx.x * 256 + threadIdx.x; t < total; t += gridDim.x * 256) {
    const uint32_t r = t / cpr, c = 8 * (t - r * cpr);
    float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* base = P + (int64_t)r * ldp + c;
    for (int s0 = 0; s0 < tp; s0 += 8) {
      f32x4_t v[8][2];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (s0 + k < tp) {
          const float* p = base + (int64_t)(s0 + k) * shard_stride;
          v[k][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
          v[k][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (s0 + k < tp) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            z[e] += v[k][0][e];
            z[4 + e] += v[k][1][e];
          }
        }
      }
    }
    const uint32_t keep = keep8((uint64_t)(row0 + r) * (uint64_t)h + (uint64_t)c, seed, thr);
    float o[8];
    unpack8(*reinterpret_cast<const u32x4_t*>(res + (int64_t)r * ldr + c), o);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += ((keep >> e) & 1u) ? z[e] * scale : 0.0f;
    *reinterpret_cast<u32x4_t*>(out + (int64_t)r * ldo + c) = pack8(o);
  }
}

// dZ[r] = Dropout'(dOut[r]) = kept ? dOut * scale : 0, for rows of this GPU's
// block (global row row0 + r), written where the caller points: its rows of
// the gathered [T, h] gradient.
__global__ void __launch_bounds__(256) sp_dropout_bwd_kernel(const bf16_t* __restrict__ dOut, int64_t ldi, int rows,
                                                             int h, uint32_t thr, float scale, uint64_t seed,
                                                             int64_t row0, bf16_t* __restrict__ dZ, int64_t ldz) {
  const uint32_t cpr = (uint32_t)h >> 3;
  const uint32_t total = (uint32_t)rows * cpr;  // < 2^31, checked on the host
  for (uint32_t t = blockIdx.x * 256 + threadIdx.x; t < total; t += gridDim.x * 256) {
    const uint32_t r = t / cpr, c = 8 * (t - r * cpr);
    const uint32_t keep = keep8((uint64_t)(row0 + r) * (uint64_t)h + (uint64_t)c, seed, thr);
    float d[8];
    unpack8(*reinterpret_cast<const u32x4_t*>(dOut + (int64_t)r * ldi + c), d);
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = ((keep >> e) & 1u) ? d[e] * scale : 0.0f;
    *reinterpret_cast<u32x4_t*>(dZ + (int64_t)r * ldz + c) = pack8(d);
  }
}

}  // namespace tpmlp
