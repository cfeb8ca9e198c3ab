// MFMA GEMM core of libtpmlp for gfx950 (CDNA4), with fused epilogues.
//
// C[M,N] = sum_k A(m,k) B(k,n) for fp32 storage, fp32 accumulate, on
// v_mfma_f32_32x32x2_f32.  (The bf16 products have kernels of their own,
// gemm_bf16.hpp and gemm_w4.hpp; the enums and tile mapping here serve all.)
//
// Operand orientation is a template choice, so one kernel body serves all
// products of the block and its backward (Y = X W; dX = dY W^T; dW = X^T dY):
//   A_KMAJ: A(m,k) = A[m*lda + k]  (rows along K, e.g. X)   else A[k*lda + m]
//   B_KMAJ: B(k,n) = B[n*ldb + k]  (e.g. W^T read from W)   else B[k*ldb + n]
//
// Data path per K step of BK = 8 chunks of 16 bytes:
//   global --16-byte loads--> registers --(transpose 8x8 if MN-major)-->
//   LDS (K-contiguous rows, XOR-swizzled, double-buffered) --ds_read_b128-->
//   MFMA.  The next K step's global loads are issued before the current
//   step's MFMAs, so HBM/L2 latency hides behind matrix work, and one
//   barrier per K step separates the two LDS buffers.
#pragma once

#include "common.hpp"

namespace tpmlp {

enum EpiKind {
  kEpiF32 = 0,        // fp32 C
  kEpiBiasAct = 1,    // Y = Act(acc + bias), H = acc + bias
  kEpiActBwd = 2,     // Y = acc * Act'(H), per-tile column sums
  kEpiSwiGLU = 3,     // packed gate/up columns: Y = silu(gate) * up (N/2 columns), H = acc (packed)
  kEpiSwiGLUBwd = 4,  // acc = dA (N columns): Y = packed [dA * up * silu'(gate) | dA * silu(gate)], H = packed gate/up
};

struct GemmArgs {
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  int M, N, K;
  int tiles_m, tiles_n, splits;
  int k_per_split;               // multiple of BK; split s covers [s*k_per_split, min(K, ...))
  float* C; int64_t ldc;         // kEpiF32 output; split s writes C + s*split_stride
  int64_t split_stride;
  void* Y; int64_t ldy;          // typed output: activation (kEpiBiasAct, kEpiSwiGLU) or gradient
                                 // (kEpiActBwd, kEpiSwiGLUBwd)
  void* H; int64_t ldh;          // typed pre-activation: written (kEpiBiasAct, kEpiSwiGLU; if non-null)
                                 // or read (kEpiActBwd, kEpiSwiGLUBwd)
  const void* bias;              // typed [N] or null (kEpiBiasAct)
  float* colsum;                 // kEpiActBwd: fp32 [tiles_m][N] per-tile column sums of dH (or null)
  int act;
  int group_m;                   // tile rows per raster group (0: 8)
  unsigned long long* clk;       // profiling: workgroup 0 writes its main loop's shader-clock
                                 // ticks and 100 MHz reference ticks here (or null)
};

// Workgroups are handed to the 8 XCDs round-robin by workgroup id.  Renumber
// them so that each XCD (with its own L2) works on a contiguous run of tiles,
// then walk tiles in groups of 8 tile-rows so that neighbours share B panels.
// pid / nwg: the workgroup's index among the nwg workgroups of this product
// (the whole grid, or one product's share of a paired launch, whose start is
// a multiple of 8 so that pid & 7 still names the XCD).
__device__ __forceinline__ void map_tile(const GemmArgs& p, int pid, int nwg, int& tm, int& tn, int& ks) {
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int per = p.tiles_m * p.tiles_n;
  ks = pid / per;
  const int t = pid - ks * per;
  const int G = p.group_m > 0 ? p.group_m : 8;
  const int width = G * p.tiles_n;
  const int gid = t / width;
  const int first = gid * G;
  const int gsz = min(p.tiles_m - first, G);
  const int r = t - gid * width;
  tm = first + r % gsz;
  tn = r / gsz;
}

__device__ __forceinline__ void map_tile(const GemmArgs& p, int& tm, int& tn, int& ks) {
  map_tile(p, (int)blockIdx.x, (int)gridDim.x, tm, tn, ks);
}

// Moves one operand tile (ROWS M- or N-indices x BK) from global memory into
// registers and from there into LDS, K-contiguous.
template <typename T, int ROWS, bool KMAJ, int NT>
struct TileLoader {
  static constexpr int EPC = Elem<T>::kPerChunk;
  static constexpr int G = ROWS / EPC;                       // 16-byte groups along MN
  static constexpr int UNITS = KMAJ ? ROWS * 8 : G * 8;      // chunks, or EPC x EPC blocks
  static constexpr int PER = (UNITS + NT - 1) / NT;
  static constexpr bool EXACT = (UNITS % NT) == 0;
  static constexpr int REGS = KMAJ ? PER : PER * EPC;
  u32x4_t r[REGS];

  __device__ __forceinline__ void load(const T* __restrict__ g, int64_t ld, int mn0, int mn_lim,
                                       int k0, int k_lim, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = u * NT + tid;
      const bool in_units = EXACT || idx < UNITS;
      if constexpr (KMAJ) {
        const int row = idx >> 3, c = idx & 7;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (in_units && (mn0 + row < mn_lim) && (k0 + c * EPC < k_lim))
          v = *reinterpret_cast<const u32x4_t*>(g + (int64_t)(mn0 + row) * ld + (k0 + c * EPC));
        r[u] = v;
      } else {
        const int gi = idx % G, c = idx / G;
        const bool okc = in_units && (mn0 + gi * EPC < mn_lim);
#pragma unroll
        for (int j = 0; j < EPC; ++j) {
          const int k = k0 + c * EPC + j;
          u32x4_t v = {0u, 0u, 0u, 0u};
          if (okc && k < k_lim)
            v = *reinterpret_cast<const u32x4_t*>(g + (int64_t)k * ld + (mn0 + gi * EPC));
          r[u * EPC + j] = v;
        }
      }
    }
  }

  __device__ __forceinline__ void store(u32x4_t* __restrict__ s, int tid) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = u * NT + tid;
      if (!(EXACT || idx < UNITS)) continue;
      if constexpr (KMAJ) {
        const int row = idx >> 3, c = idx & 7;
        s[row * 8 + swz(row, c)] = r[u];
      } else {
        const int gi = idx % G, c = idx / G;
        const u32x4_t* in = &r[u * EPC];
#pragma unroll
        for (int m = 0; m < EPC; ++m) {
          u32x4_t t;
          if constexpr (EPC == 8) {
            // bf16: word q of chunk m packs k = 2q (low half) and 2q + 1 (high half) of column m.
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t a = in[2 * q][m >> 1], b = in[2 * q + 1][m >> 1];
              t[q] = (m & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) t[q] = in[q][m];
          }
          const int row = gi * EPC + m;
          s[row * 8 + swz(row, c)] = t;
        }
      }
    }
  }
};

template <typename T> struct Mfma;   // fp32 only: bf16 products run on gemm_bf16.hpp and gemm_w4.hpp
template <> struct Mfma<float> {
  // Four 32x32x2 products, one per float of the lane's 4-float chunk.  Each
  // lane group (lane / 32) takes the same K entries for A and B, so the four
  // products cover the 8 K values of the two chunks once each.
  static __device__ __forceinline__ void step(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc, 0, 0, 0);
  }
};

// One workgroup computes a BM x BN tile with WGM x WGN waves; each wave owns a
// (BM/WGM) x (BN/WGN) sub-tile made of 32x32 MFMA blocks.  Accumulator lane
// layout of a 32x32 block: lane l, register v holds row 8*(v/4) + 4*(l/32) + v%4,
// column l%32.
template <typename T, int BM, int BN, int WGM, int WGN, bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_kernel(const GemmArgs p) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int BK = 8 * EPC;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int STAGE = (BM + BN) * 8;  // chunks per LDS stage
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");

  __shared__ u32x4_t lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  int tmi, tni, ks;
  map_tile(p, tmi, tni, ks);
  const int m0 = tmi * BM, n0 = tni * BN;
  const int kbeg = ks * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  const T* __restrict__ A = static_cast<const T*>(p.A);
  const T* __restrict__ B = static_cast<const T*>(p.B);
  TileLoader<T, BM, A_KMAJ, NT> la;
  TileLoader<T, BN, B_KMAJ, NT> lb;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  if (nk > 0) {
    la.load(A, p.lda, m0, p.M, kbeg, kend, tid);
    lb.load(B, p.ldb, n0, p.N, kbeg, kend, tid);
    la.store(lds, tid);
    lb.store(lds + BM * 8, tid);
    __syncthreads();
  }

  const int lrow = lane & 31;
  const int lchunk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = kbeg + (kt + 1) * BK;
      la.load(A, p.lda, m0, p.M, k0, kend, tid);
      lb.load(B, p.ldb, n0, p.N, k0, kend, tid);
    }
    const u32x4_t* cA = lds + cur * STAGE;
    const u32x4_t* cB = cA + BM * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int chunk = 2 * s + lchunk;
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WTM + i * 32 + lrow;
        af[i] = cA[row * 8 + swz(row, chunk)];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WTN + j * 32 + lrow;
        bfr[j] = cB[row * 8 + swz(row, chunk)];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<T>::step(acc[i][j], af[i], bfr[j]);
    }
    if (more) {
      u32x4_t* nA = lds + (cur ^ 1) * STAGE;
      la.store(nA, tid);
      lb.store(nA + BM * 8, tid);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue --
  const int M = p.M, N = p.N;
  if constexpr (EPI == kEpiF32) {
    float* __restrict__ C = p.C + (int64_t)ks * p.split_stride;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WTN + j * 32 + lrow;
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lchunk + (v & 3);
          if (row < M) C[(int64_t)row * p.ldc + col] = acc[i][j][v];
        }
    }
  } else if constexpr (EPI == kEpiBiasAct) {
    T* __restrict__ Y = static_cast<T*>(p.Y);
    T* __restrict__ Hs = static_cast<T*>(p.H);
    const T* __restrict__ bias = static_cast<const T*>(p.bias);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WTN + j * 32 + lrow;
      if (col >= N) continue;
      const float bv = bias ? Elem<T>::load(bias + col) : 0.0f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lchunk + (v & 3);
          if (row < M) {
            const float hv = acc[i][j][v] + bv;
            if (Hs) Elem<T>::store(Hs + (int64_t)row * p.ldh + col, hv);
            Elem<T>::store(Y + (int64_t)row * p.ldy + col, act_apply(p.act, hv));
          }
        }
    }
  } else {  // kEpiActBwd: dH = acc * Act'(H), plus per-tile column sums of dH
    T* __restrict__ Y = static_cast<T*>(p.Y);
    const T* __restrict__ Hs = static_cast<const T*>(p.H);
    float* red = reinterpret_cast<float*>(lds);  // [WGM][BN]
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WTN + j * 32 + lrow;
      float cs = 0.0f;
      if (col < N) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lchunk + (v & 3);
            if (row < M) {
              // H is read only for the GeLU derivative: with no activation it may be NULL.
              const float d = p.act == kActGeluTanh
                                  ? acc[i][j][v] * gelu_tanh_grad(Elem<T>::load(Hs + (int64_t)row * p.ldh + col))
                                  : acc[i][j][v];
              Elem<T>::store(Y + (int64_t)row * p.ldy + col, d);
              cs += d;
            }
          }
      }
      cs += __shfl_xor(cs, 32);
      if (lchunk == 0) red[wm * BN + wn * WTN + j * 32 + lrow] = cs;
    }
    if (p.colsum) {
      __syncthreads();
      for (int c = tid; c < BN; c += NT) {
        if (n0 + c >= N) continue;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WGM; ++w) s += red[w * BN + c];
        p.colsum[(int64_t)tmi * N + n0 + c] = s;
      }
    }
  }
}

}  // namespace tpmlp
