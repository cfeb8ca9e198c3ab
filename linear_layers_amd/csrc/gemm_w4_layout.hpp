// LDS layout of the four-wave bf16 GEMM tiles (gemm_w4.hpp), K steps of 64:
// where each 16-byte chunk of an operand tile sits in LDS and which bytes each
// lane's MFMA fragment reads come from.  Plain integer functions, callable on
// the host, so that the layouts, the fragment contents and the bank pattern
// are checked on the CPU over every lane (tests/test_gemm_layout_cpu.py).
//
// Bank model (64 banks of 4 bytes), fitted to rocprofv3's bank-conflict
// counts for ten probe patterns of ds_read_b128 (linear, strided, and the
// fragment reads of both GEMM variants): a ds_read_b128 is served 16 lanes
// per cycle, lanes 8..23, then 0..7 with 24..31, then the same two groups
// of lanes 32..63; the layouts below are also conflict-free under every
// other grouping that fits those counts.  A ds_read_b64_tr_b16 is served
// 32 lanes per cycle (lanes 0..31, then 32..63; it measured conflict-free).
#pragma once

#if !defined(__HIPCC__) && !defined(__host__)
#define __host__
#define __device__
#endif

#include <stdint.h>

namespace tpmlp {
namespace w4 {

// K-contiguous tile: rows of 8 chunks of 16 bytes.  Chunk c of row r sits at
// position c ^ swz_k(r), swz_k taking bits 1, 3, 2 of r to bits 0, 1, 2.  A
// fragment read puts 16 rows at one chunk (4 chunks over the lane groups)
// through the cycles; a 128-byte row covers half of the banks, and swz_k
// spreads the rows of each parity over distinct 16-byte bank groups in every
// cycle.  An involution in c.
__host__ __device__ constexpr int swz_k(int r) {
  return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2);
}
__host__ __device__ constexpr int pos_k(int r, int c) { return c ^ swz_k(r); }

// M/N-contiguous tile of qpr chunks per K-row: position of chunk q of K-row
// k.  A transposing read cycle (32 lanes) takes 32 bytes (a chunk pair) from
// each of 8 K-rows, k0..k0+3 and k0+8..k0+11 (k0 a multiple of 4), which must
// land on the 8 distinct 32-byte bank groups of a 256-byte bank line.
//   * qpr a multiple of 16 (K-row pitch a multiple of 256 bytes): XOR with
//     4 (k & 3) + 2 bit3(k), below 16, so the map stays inside q's aligned
//     group of 16 chunks.
//   * qpr = 8 (mod 16) (pitch 128 bytes more than a multiple of 256): odd
//     K-rows sit half a bank line further, so bit 0 of k already splits the
//     rows in two; XOR with 4 bit1(k) + 2 bit3(k), below 8, separates the 4
//     rows of each parity and stays inside q's aligned group of 8 chunks.
// Both are involutions in q and keep chunk pairs (2a, 2a + 1) together.
__host__ __device__ constexpr int pos_t(int qpr, int k, int q) {
  return (qpr & 15) == 0 ? q ^ ((k & 3) << 2) ^ (((k >> 3) & 1) << 1)
                         : q ^ (((k >> 1) & 1) << 2) ^ (((k >> 3) & 1) << 1);
}

// Byte offset, in a K-contiguous tile, of the 16 bytes lane `lane` reads for
// fragment block f (16 rows from the wave's first row w0) of K substep s:
// row w0 + 16 f + (lane & 15), K values 32 s + 8 (lane >> 4) .. + 7.
__host__ __device__ constexpr uint32_t frag_k(int w0, int lane, int f, int s) {
  const int row = w0 + 16 * f + (lane & 15);
  const int c = 4 * s + (lane >> 4);
  return (uint32_t)(row * 128 + pos_k(row, c) * 16);
}

// The same offset as the kernel forms it: with w0 a multiple of 16 the
// swizzle depends on lane & 15 only, so one base per substep and an
// immediate f * 2048 serve every fragment.
__host__ __device__ constexpr uint32_t frag_k_base(int w0, int lane, int s) { return frag_k(w0, lane, 0, s); }
__host__ __device__ constexpr uint32_t frag_k_fast(int w0, int lane, int f, int s) {
  return frag_k_base(w0, lane, s) + (uint32_t)(f * 2048);
}

// Byte offset, in an M/N-contiguous tile (qpr chunks per K-row), of the 8
// bytes lane `lane` addresses in transposing read r (0, 1) of fragment block
// f (16 columns from the wave's first column w0), substep s.  The 16-lane
// group g = lane >> 4 addresses K-rows 32 s + 8 g + 4 r + j / 4 (j = lane & 15)
// at column w0 + 16 f + 4 (j & 3); ds_read_b64_tr_b16 then hands lane j the
// K values 32 s + 8 g + 4 r .. + 3 of column w0 + 16 f + j.
__host__ __device__ constexpr uint32_t frag_t(int qpr, int w0, int lane, int f, int s, int r) {
  const int g = lane >> 4, j = lane & 15;
  const int k = 32 * s + 8 * g + 4 * r + (j >> 2);
  const int col = w0 + 16 * f + 4 * (j & 3);
  return (uint32_t)(k * qpr * 16 + pos_t(qpr, k, col >> 3) * 16 + (col & 7) * 2);
}
// As the kernel forms it: one base per block f (substep 0, read 0), the rest
// an immediate (32 s + 4 r) K-rows further (bits 0, 1 and 3 of k do not
// depend on s or r).
__host__ __device__ constexpr uint32_t frag_t_fast(int qpr, int w0, int lane, int f, int s, int r) {
  return frag_t(qpr, w0, lane, f, 0, 0) + (uint32_t)((32 * s + 4 * r) * qpr * 16);
}

}  // namespace w4
}  // namespace tpmlp
