// Eight-wave bf16 MFMA GEMM of libtpmlp for gfx950 (CDNA4): C[M,N] = sum_k
// A(m,k) B(k,n), fp32 accumulate on v_mfma_f32_32x32x16_bf16, fp32 output.
// The library runs it at one configuration only, 256x320 tiles of 8 waves as
// 4 x 2 (64x160 per wave): fp32 outputs whose width (5120) leaves 256x256
// tiles a fraction of a round short.  Every other bf16 product runs on the
// four-wave kernel (gemm_w4.hpp), which shares this file's tile helpers.
//
// Operand orientation (template flags), as in the products of the block:
//   A_KMAJ: A(m,k) = A[m*lda + k]   else A(m,k) = A[k*lda + m]
//   B_KMAJ: B(k,n) = B[n*ldb + k]   else B(k,n) = B[k*ldb + n]
//
// Data path, per K step of 32:
//   * Both tiles go from global memory straight into LDS with
//     buffer_load_dwordx4 ... lds (no VGPR staging, no ds_write).  The buffer
//     descriptor is re-based per tile so rows past the end of an operand read
//     as zero; a K-contiguous tile whose last K step is partial gets its
//     out-of-range chunks zeroed in LDS.
//   * A K-contiguous tile is stored as rows of 4 x 16-byte chunks along K
//     (chunk c of row r at position c ^ ((r >> 2) & 3)) and read with
//     ds_read_b128: one read gives a lane 8 consecutive K values.
//   * An M/N-contiguous tile is stored as 32 K-rows of BM (or BN) elements
//     (16-byte chunk q of K-row k at position q ^ 4*(k&3); in a row whose
//     chunk count is not a multiple of 16, the last 8 chunks at q ^ 4*(k&1))
//     and read with ds_read_b64_tr_b16, which transposes 4x4 blocks of 16-bit
//     values across groups of 16 lanes, so two reads give a lane its 8 K values.
//   * The MFMA takes the B fragment as its first operand and the A fragment
//     as its second, so each lane's accumulators hold 4 consecutive output
//     columns of one row, which the epilogue stores as 8- or 16-byte vectors.
//   * NS LDS stages form a ring: the loads of step k+NS-1 are issued at the
//     start of step k, so NS-1 steps of data are in flight behind the MFMAs
//     (one wave per SIMD cannot hide memory latency any other way).  Each
//     step has one barrier, in its middle: after it the first fragments of
//     step k+1 are read while the second half of step k's MFMAs runs.
//   * The stages are separate LDS objects indexed at compile time (the loop
//     is unrolled NS times), so the compiler can tell in-flight loads into
//     one stage from reads of another.  Trailing steps up to a multiple of NS
//     are zero-filled stages, so the loop body carries no MFMA under a branch.
#pragma once

#include "common.hpp"
#include <type_traits>

#include "gemm.hpp"  // GemmArgs, EpiKind, map_tile

namespace tpmlp {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int waitcnt_vm(int n) { return 0x0f70 | (n & 0xf) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xc07f;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // v_cvt_pk_bf16_f32 rounds to nearest even.
  const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ROWS (M or N) x BKT (K) operand tile; NF fragment blocks of 32 rows per wave.
template <int ROWS, bool KMAJ, int BKT, int NW = 4, int NF = 4>
struct Bf16Tile {
  // One operand tile of ROWS (M or N) x BKT (K) bf16 = ROWS * BKT * 2 bytes.
  static constexpr int CPR = BKT / 8;           // 16-byte chunks per K-contiguous row
  static constexpr int BYTES = ROWS * BKT * 2;
  static constexpr int SLOTS = ROWS * CPR;      // 16-byte slots
  static constexpr int INSTR = SLOTS / (64 * NW);  // buffer loads per wave
  static constexpr int QPR = ROWS / 8;          // chunks per K-row (M/N-contiguous layout)
  static constexpr int QPR16 = QPR & ~15;       // chunks under the 4-row swizzle; the rest (8) under a 2-row one
  static constexpr int NFB = KMAJ ? 4 : (NF > 4 ? NF : 4);
  static_assert(BKT == 32 || BKT == 64, "K step of 32 or 64");
  static_assert(SLOTS % (64 * NW) == 0, "tile too small for the waves");
  static_assert(KMAJ || (ROWS >= 128 && (QPR - QPR16 == 0 || QPR - QPR16 == 8)),
                "the K-row swizzle needs at least 16 chunks per K-row, in groups of 16 and at most one of 8");

  uint32_t voff[INSTR];   // per-lane byte offsets in the re-based buffer
  uint32_t fbase[NFB];    // per-lane LDS offsets of the MFMA fragments

  // Position of 16-byte chunk q of K-row k in an M/N-contiguous tile: an XOR
  // that stays inside q's group of 16 chunks (or the trailing group of 8), so
  // it is an involution on the row.
  static __device__ __forceinline__ int swz_t(int k, int q) {
    return q < QPR16 ? q ^ ((k & 3) << 2) : q ^ ((k & 1) << 2);
  }

  // Position of chunk c of row r in a K-contiguous tile: conflict-free for
  // one row written as CPR chunks and for 16 consecutive rows read at one chunk.
  static __device__ __forceinline__ int pos_k(int r, int c) {
    if constexpr (CPR == 4) return c ^ ((r >> 2) & 3);
    else return c ^ (r & 7) ^ ((r >> 3) & 7);
  }

  __device__ __forceinline__ void init(int wave, int lane, int64_t ld, int w0) {
#pragma unroll
    for (int j = 0; j < INSTR; ++j) {
      const int s = (wave * INSTR + j) * 64 + lane;
      if constexpr (KMAJ) {
        const int row = s / CPR, c = pos_k(row, s % CPR);   // pos_k is an involution in c
        voff[j] = (uint32_t)(((int64_t)row * ld + c * 8) * 2);
      } else {
        const int k = s / QPR, q = swz_t(k, s % QPR);
        voff[j] = (uint32_t)(((int64_t)k * ld + q * 8) * 2);
      }
    }
    // Fragment rows are w0 + 32 f + (lane & 31) with w0 a multiple of 32.
    if constexpr (KMAJ) {
      const uint32_t lb = (uint32_t)(w0 + (lane & 31)) * (uint32_t)(CPR * 16);
      if constexpr (CPR == 4) {
        // chunk 2S + lane/32 at (2S + lane/32) ^ (((lane & 31) >> 2) & 3): one base per S
        const int x = ((lane & 31) >> 2) & 3;
#pragma unroll
        for (int S = 0; S < 2; ++S) fbase[S] = lb + (uint32_t)(((2 * S + (lane >> 5)) ^ x) << 4);
        fbase[2] = fbase[3] = 0;
      } else {
        // chunk 2S + lane/32 of row r at (2S + lane/32) ^ (r & 7) ^ ((r >> 3) & 7); with
        // r = w0 + 32 f + (lane & 31) the XOR term is L ^ 4 (f & 1) (L takes the
        // parity of w0 / 32), so the bases are indexed by X = (2S ^ 4(f&1)) / 2.
        const int L = (lane >> 5) ^ (lane & 7) ^ ((lane & 31) >> 3) ^ (((w0 >> 5) & 1) << 2);
#pragma unroll
        for (int x = 0; x < 4; ++x) fbase[x] = lb + (uint32_t)((L ^ (2 * x)) << 4);
      }
    } else {
      // 16-lane group g reads K-rows kb + j/4 (j = lane & 15) at column
      // w0 + 32 f + 16 (g&1) + 4 (j&3); the transpose hands lane j the 4 K
      // values of column w0 + 32 f + 16 (g&1) + j.  (k & 3) = j >> 2.  The
      // four chunks of fragment f start at a multiple of 4, in one swizzle group.
      const int g = lane >> 4, j = lane & 15;
      const int qlow = 2 * (g & 1) + ((j & 3) >> 1);
      const int kl = 8 * (g >> 1) + (j >> 2);
#pragma unroll
      for (int f = 0; f < NFB; ++f) {
        const int qb = (w0 >> 3) + 4 * f;
        const int x = qb < QPR16 ? (j & 12) : (j & 4);
        fbase[f] = (uint32_t)((kl * QPR + ((qb ^ x) | qlow)) * 16 + (j & 1) * 8);
      }
    }
  }

  // Issue this wave's loads of one K step into `dst`; base/nbytes describe the
  // re-based buffer (bytes past nbytes read as zero).  The loads are written
  // as inline asm so that the compiler does not track them: it would
  // otherwise add a full vmcnt(0) drain before reads of other LDS stages at
  // the loop head.  The kernel waits for them itself (vmcnt before each
  // barrier, and a full drain after the loop); the compiler's own waits stay
  // correct because loads it does not count can only make them wait longer.
  __device__ __forceinline__ void load(const bf16_t* base, uint32_t nbytes, lds_char* dst, int wave) const {
    const uint64_t addr = reinterpret_cast<uint64_t>(base);
    const i32x4_t rsrc = {(int)(uint32_t)addr, (int)((addr >> 32) & 0xffffu), (int)nbytes, kBufferWord3};
#pragma unroll
    for (int j = 0; j < INSTR; ++j) {
      const uint32_t lds = (uint32_t)(uintptr_t)(dst + (wave * INSTR + j) * 1024);
      // m0 is set and consumed inside this one statement; no compiler-generated
      // instruction uses m0 (tests/test_m0_invariant_cpu.py checks the built library).
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :
                   : "s"(lds), "v"(voff[j]), "s"(rsrc)
                   : "memory", "m0");
    }
  }

  // Zero this wave's slots of the tile (a step past the end of K).
  __device__ __forceinline__ void zero(lds_char* dst, int wave, int lane) const {
#pragma unroll
    for (int j = 0; j < INSTR; ++j)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(dst + ((wave * INSTR + j) * 64 + lane) * 16) =
          u32x4_t{0u, 0u, 0u, 0u};
  }

  // K-contiguous tiles: zero the chunks at K offset >= kvalid (last, partial step).
  __device__ __forceinline__ void zero_tail(lds_char* dst, int wave, int lane, int kvalid) const {
    static_assert(KMAJ, "only K-contiguous tiles need the fix-up");
#pragma unroll
    for (int j = 0; j < INSTR; ++j) {
      const int s = (wave * INSTR + j) * 64 + lane;
      const int row = s / CPR, c = pos_k(row, s % CPR);
      if (c * 8 >= kvalid)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(dst + s * 16) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // 8 K values (k = 16 S + 8 (lane/32) + t, t = 0..7) of fragment block F.
  template <int F, int S>
  __device__ __forceinline__ u32x4_t frag(const lds_char* src) const {
    if constexpr (KMAJ) {
      constexpr int X = CPR == 4 ? S : (((2 * S) ^ (4 * (F & 1))) >> 1);
      return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(src + fbase[X] + F * 32 * CPR * 16);
    } else {
      static_assert(F < NFB, "too many fragment blocks");
      const lds_char* p0 = src + fbase[F] + 16 * S * QPR * 16;
      const lds_char* p1 = p0 + 4 * QPR * 16;
      const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p0);
      const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p1);
      const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0);
      const u32x2_t w1 = __builtin_bit_cast(u32x2_t, v1);
      return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
    }
  }
};

// Reads fragments F..NF-1 of one tile for K-substep S (compile-time indices,
// so every LDS offset is an immediate).
template <int F, int NF, int S>
struct FragLoop {
  template <class Tile>
  __device__ __forceinline__ static void run(const Tile& t, const lds_char* src, u32x4_t* out) {
    out[F] = t.template frag<F, S>(src);
    FragLoop<F + 1, NF, S>::run(t, src, out);
  }
};
template <int NF, int S>
struct FragLoop<NF, NF, S> {
  template <class Tile>
  __device__ __forceinline__ static void run(const Tile&, const lds_char*, u32x4_t*) {}
};

// One workgroup's tile: workgroup pid of the nwg that compute product p.
template <int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI, int NS, int OCC, int BKT, int WGN, int WGM>
__device__ __forceinline__ void gemm_bf16_body(const GemmArgs& p, int pid, int nwg) {
  constexpr int NW = WGM * WGN;  // WGM x WGN waves
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM * 32 * WGM == BM && FN * 32 * WGN == BN, "wave tiles of whole 32x32 blocks");
  constexpr int NSUB = BKT / 16;             // MFMA K-substeps per step
  using TA = Bf16Tile<BM, A_KMAJ, BKT, NW, FM>;
  using TB = Bf16Tile<BN, B_KMAJ, BKT, NW, FN>;
  constexpr int STAGE = TA::BYTES + TB::BYTES;
  constexpr int LPS = TA::INSTR + TB::INSTR;  // buffer loads per wave per step
  static_assert(NS >= 2 && NS <= 6, "2..6 stages");
  static_assert(NS * STAGE * OCC <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char st3[NS > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char st4[NS > 4 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char st5[NS > 5 ? STAGE : 16];
  auto stage = [&](auto I) -> lds_char* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return (lds_char*)st0;
    else if constexpr (i == 1) return (lds_char*)st1;
    else if constexpr (i == 2) return (lds_char*)st2;
    else if constexpr (i == 3) return (lds_char*)st3;
    else if constexpr (i == 4) return (lds_char*)st4;
    else return (lds_char*)st5;
  };
  (void)stage;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // Profiling only: the shader clock over workgroup 0's main loop.
  unsigned long long clk0 = 0, ref0 = 0;
  if (p.clk != nullptr && pid == 0) {
    clk0 = __builtin_amdgcn_s_memtime();
    ref0 = __builtin_amdgcn_s_memrealtime();
  }

  int tmi, tni, ks;
  map_tile(p, pid, nwg, tmi, tni, ks);
  const int m0 = tmi * BM, n0 = tni * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int kbeg = ks * p.k_per_split;
  const int kend = min(K, kbeg + p.k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + BKT - 1) / BKT : 0;
  const int nkp = ((nk + NS - 1) / NS) * NS;  // padded with zero-filled steps
  const int ktail = (kend - kbeg) & (BKT - 1);  // valid K in the last real step (0 = full)

  const bf16_t* A = static_cast<const bf16_t*>(p.A);
  const bf16_t* B = static_cast<const bf16_t*>(p.B);
  TA ta;
  TB tb;
  ta.init(wave, lane, p.lda, wm * WTM);
  tb.init(wave, lane, p.ldb, wn * WTN);

  // Re-based buffers of step kt (bytes past nbytes read as zero).
  auto bases = [&](int kt, const bf16_t*& pa, uint32_t& na, const bf16_t*& pb, uint32_t& nb) {
    const int k0 = kbeg + kt * BKT;
    if constexpr (A_KMAJ) {
      const int rows = min(BM, M - m0);
      na = (uint32_t)(((int64_t)(rows - 1) * p.lda + (kend - k0)) * 2);
      pa = A + (int64_t)m0 * p.lda + k0;
    } else {
      const int kv = min(BKT, kend - k0);
      na = (uint32_t)(((int64_t)(kv - 1) * p.lda + (M - m0)) * 2);
      pa = A + (int64_t)k0 * p.lda + m0;
    }
    if constexpr (B_KMAJ) {
      const int rows = min(BN, N - n0);
      nb = (uint32_t)(((int64_t)(rows - 1) * p.ldb + (kend - k0)) * 2);
      pb = B + (int64_t)n0 * p.ldb + k0;
    } else {
      const int kv = min(BKT, kend - k0);
      nb = (uint32_t)(((int64_t)(kv - 1) * p.ldb + (N - n0)) * 2);
      pb = B + (int64_t)k0 * p.ldb + n0;
    }
  };
  // Step kt's tiles into stage `dst`: loads for real steps, zeros past the end.
  auto issue = [&](int kt, lds_char* dst) {
    if (kt < nk) {
      const bf16_t* pa;
      const bf16_t* pb;
      uint32_t na, nb;
      bases(kt, pa, na, pb, nb);
      ta.load(pa, na, dst, wave);
      tb.load(pb, nb, dst + TA::BYTES, wave);
    } else if (kt < nkp) {
      ta.zero(dst, wave, lane);
      tb.zero(dst + TA::BYTES, wave, lane);
    }
  };

  // The same loads in two halves (A, then B), for the split below; steps past
  // the end of K zero both tiles in the first half.
  auto issue_a = [&](int kt, lds_char* dst) {
    if (kt < nk) {
      const bf16_t* pa;
      const bf16_t* pb;
      uint32_t na, nb;
      bases(kt, pa, na, pb, nb);
      ta.load(pa, na, dst, wave);
    } else if (kt < nkp) {
      ta.zero(dst, wave, lane);
      tb.zero(dst + TA::BYTES, wave, lane);
    }
  };
  auto issue_b = [&](int kt, lds_char* dst) {
    if (kt < nk) {
      const bf16_t* pa;
      const bf16_t* pb;
      uint32_t na, nb;
      bases(kt, pa, na, pb, nb);
      tb.load(pb, nb, dst + TA::BYTES, wave);
    }
  };
  // Wait until this wave's loads of step `next` have landed: the loads of
  // the real steps after it that are already issued (at most NS-2) may stay
  // in flight.
  auto wait_landed = [&](int next) {
    const int later = min(NS - 2, max(0, nk - 1 - next));
    switch (later) {
      case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(1 * LPS)); break;
      case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPS)); break;
      case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * LPS)); break;
      default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * LPS)); break;
    }
  };
  auto fix_tail = [&](int kt, lds_char* dst) {
    if (kt == nk - 1 && ktail != 0) {
      if constexpr (A_KMAJ) ta.zero_tail(dst, wave, lane, ktail);
      if constexpr (B_KMAJ) tb.zero_tail(dst + TA::BYTES, wave, lane, ktail);
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto mfmas = [&](const u32x4_t (&af)[FM], const u32x4_t (&bfr)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bfr[j]),
                                                            __builtin_bit_cast(bf16x8_t, af[i]), acc[i][j], 0, 0, 0);
  };

  u32x4_t a0[FM], b0[FN], a1[FM], b1[FN];  // fragments of even / odd K-substeps

  // With K steps of 64 the next substep's LDS reads are spread between the
  // current substep's MFMAs instead of going out as one burst (which filled
  // the LDS command queue), in the order the MFMAs use them: A block 0, the
  // B blocks, the other A blocks; a transposing fragment is two reads.
  // (Measured: 1-4% faster on the tile shapes with K steps of 64, neutral on
  // 256x192; the 256x320 weight gradient, both operands through transposing
  // reads, ran 2.7% slower inside the attention block, and 256x256 tiles with
  // K steps of 32 ran slower in isolation: those keep the burst.)
  constexpr bool kIlv = BKT == 64 && !(BN == 320 && !A_KMAJ && !B_KMAJ);
  // Weight gradients (both operands through transposing reads; 256x256 and
  // 128x128 tiles) also issue the next step's B loads one substep after its
  // A loads (measured 2-5% faster in isolation; input gradients measured
  // slower so).  With two stages every wait for a step's loads is a full
  // vmcnt(0), so the split leaves the load accounting as it is.
  constexpr bool kSplit = kIlv && !A_KMAJ && !B_KMAJ;
  static_assert(!kSplit || NS == 2, "the split loads assume two stages");
  auto rd = [&](auto SC, const lds_char* src, u32x4_t (&af)[FM], u32x4_t (&bfr)[FN]) {
    constexpr int S = decltype(SC)::value;
    FragLoop<0, 1, S>::run(ta, src, af);
    FragLoop<0, FN, S>::run(tb, src + TA::BYTES, bfr);
    FragLoop<1, FM, S>::run(ta, src, af);
  };
  auto ilv = [&]() {
    constexpr int nds = FM * (A_KMAJ ? 1 : 2) + FN * (B_KMAJ ? 1 : 2);   // LDS reads of one substep
    constexpr int slots = FM * FN - 2;   // the last two MFMAs give the last reads time to land
    static_assert(!kIlv || slots >= 1, "at least three MFMAs per substep");
    constexpr int per = slots >= 1 ? (nds + slots - 1) / slots : nds;
    constexpr int full = nds / per, rest = nds - full * per;   // groups of `per` reads, then one of `rest`
#pragma unroll
    for (int i = 0; i < full; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, per, 0);   // then `per` LDS reads
    }
    if constexpr (rest > 0) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, rest, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - full - (rest > 0 ? 1 : 0), 0);
  };

  // One step in stage ST (compile time) with its substep-0 fragments in
  // a0/b0.  Order (kept by the scheduling barriers): loads of step kt+NS-1;
  // then for each substep s the reads of substep s+1 go out before (kIlv:
  // between) the MFMAs of substep s; before the last substep's MFMAs the kernel waits for step
  // kt+1, passes the barrier and reads that step's substep-0 fragments.
  auto step = [&](auto STc, int kt) {
    constexpr int ST = decltype(STc)::value;
    lds_char* cur = stage(STc);
    lds_char* nxt = stage(std::integral_constant<int, (ST + 1) % NS>{});
    lds_char* const ahead = stage(std::integral_constant<int, (ST + NS - 1) % NS>{});
    if constexpr (kSplit) {
      if (kt + NS - 1 < nkp) issue_a(kt + NS - 1, ahead);
    } else {
      if (kt + NS - 1 < nkp) issue(kt + NS - 1, ahead);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kIlv) {
      rd(std::integral_constant<int, 1>{}, cur, a1, b1);
      mfmas(a0, b0);
      ilv();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kSplit) {
        if (kt + NS - 1 < nkp) issue_b(kt + NS - 1, ahead);
        __builtin_amdgcn_sched_barrier(0);
      }
      rd(std::integral_constant<int, 2>{}, cur, a0, b0);
      mfmas(a1, b1);
      ilv();
      __builtin_amdgcn_sched_barrier(0);
      rd(std::integral_constant<int, 3>{}, cur, a1, b1);
      mfmas(a0, b0);
      ilv();
      __builtin_amdgcn_sched_barrier(0);
    } else {
      FragLoop<0, FM, 1>::run(ta, cur, a1);
      FragLoop<0, FN, 1>::run(tb, cur + TA::BYTES, b1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NSUB == 4) {
        FragLoop<0, FM, 2>::run(ta, cur, a0);
        FragLoop<0, FN, 2>::run(tb, cur + TA::BYTES, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        FragLoop<0, FM, 3>::run(ta, cur, a1);
        FragLoop<0, FN, 3>::run(tb, cur + TA::BYTES, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(a0, b0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (kt + 1 < nkp) {
      wait_landed(kt + 1);
      fix_tail(kt + 1, nxt);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
      FragLoop<0, FM, 0>::run(ta, nxt, a0);
      FragLoop<0, FN, 0>::run(tb, nxt + TA::BYTES, b0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfmas(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
  };

  if (nk > 0) {
    // Prologue: steps 0..NS-2 in flight, step 0 landed, its first fragments read.
    issue(0, stage(std::integral_constant<int, 0>{}));
    if constexpr (NS > 2) issue(1, stage(std::integral_constant<int, 1>{}));
    if constexpr (NS > 3) issue(2, stage(std::integral_constant<int, 2>{}));
    if constexpr (NS > 4) issue(3, stage(std::integral_constant<int, 3>{}));
    if constexpr (NS > 5) issue(4, stage(std::integral_constant<int, 4>{}));
    wait_landed(0);
    fix_tail(0, stage(std::integral_constant<int, 0>{}));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    FragLoop<0, FM, 0>::run(ta, stage(std::integral_constant<int, 0>{}), a0);
    FragLoop<0, FN, 0>::run(tb, stage(std::integral_constant<int, 0>{}) + TA::BYTES, b0);
    for (int kt = 0; kt < nkp; kt += NS) {
      step(std::integral_constant<int, 0>{}, kt);
      step(std::integral_constant<int, 1>{}, kt + 1);
      if constexpr (NS > 2) step(std::integral_constant<int, 2>{}, kt + 2);
      if constexpr (NS > 3) step(std::integral_constant<int, 3>{}, kt + 3);
      if constexpr (NS > 4) step(std::integral_constant<int, 4>{}, kt + 4);
      if constexpr (NS > 5) step(std::integral_constant<int, 5>{}, kt + 5);
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // drain the loads the compiler does not see
  __syncthreads();
  if (p.clk != nullptr && pid == 0 && tid == 0) {
    p.clk[0] = __builtin_amdgcn_s_memtime() - clk0;
    p.clk[1] = __builtin_amdgcn_s_memrealtime() - ref0;
  }
  // ------------------------------------------------------------ epilogue --
  // Lane l, block (i, j), register v: row m0 + wm*WTM + 32 i + (l & 31),
  // column n0 + wn*WTN + 32 j + 8 (v/4) + 4 (l/32) + v%4.
  const int mrow = m0 + wm * WTM + (lane & 31);
  const int ncol = n0 + wn * WTN + 4 * (lane >> 5);
  static_assert(EPI == kEpiF32, "this kernel keeps the fp32 epilogue only");
  if constexpr (EPI == kEpiF32) {
    float* __restrict__ C = p.C + (int64_t)ks * p.split_stride;
    // Through LDS to whole 128-byte lines, stored non-temporally: a store
    // straight from the sums covers 32 rows x 32 bytes.  Each wave takes its
    // tile 16 rows at a time into its own region of the (now free) stages,
    // row-major with a 16-byte pad per row, and reads it back as runs of 64
    // consecutive 16-byte chunks of those rows (a row is a whole number of
    // lines: WTN * 4 bytes, a multiple of 128).
    constexpr int RB = WTN * 4 + 16;   // bytes per staged row
    static_assert((WTN * 4) % 128 == 0 && 16 * RB * (NW / 2) <= STAGE, "epilogue staging");
    static_assert((16 * WTN / 4) % 64 == 0, "whole chunk runs per wave");
    lds_char* const reg = (wave < NW / 2 ? stage(std::integral_constant<int, 0>{}) : stage(std::integral_constant<int, 1>{})) +
                          (wave % (NW / 2)) * 16 * RB;
    const int half = (lane & 31) >> 4;   // rows 0-15 or 16-31 of a 32-row block
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int hsel = 0; hsel < 2; ++hsel) {
        if (half == hsel) {
          const int r = lane & 15;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *reinterpret_cast<__attribute__((address_space(3))) f32x4_t*>(reg + r * RB + (32 * j + 8 * g + 4 * (lane >> 5)) * 4) =
                  f32x4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        const int row0 = m0 + wm * WTM + 32 * i + 16 * hsel;
        const int col0 = n0 + wn * WTN;
#pragma unroll
        for (int k = 0; k < 16 * WTN / 4 / 64; ++k) {
          const int c = 64 * k + lane;          // chunk of the 16 rows x WTN/4 chunks
          const int r = c / (WTN / 4), q = c % (WTN / 4);
          const f32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(reg + r * RB + q * 16);
          const int row = row0 + r, col = col0 + 4 * q;
          if (row < M && col < N) __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(C + (int64_t)row * p.ldc + col));
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // reads done before the next rows overwrite the region
        __builtin_amdgcn_wave_barrier();
      }
    }
    (void)mrow;
    (void)ncol;
  }
}

template <int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI, int NS, int OCC = 1, int BKT = 32, int WGN = 2,
          int WGM = 2>
__global__ void __launch_bounds__(64 * WGM * WGN, OCC)
gemm_bf16_kernel(const GemmArgs p) {
  gemm_bf16_body<BM, BN, A_KMAJ, B_KMAJ, EPI, NS, OCC, BKT, WGN, WGM>(p, (int)blockIdx.x, (int)gridDim.x);
}

}  // namespace tpmlp
