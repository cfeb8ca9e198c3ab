// Four-wave bf16 GEMM of libtpmlp for gfx950: 256x256 output tiles, one
// workgroup of 4 waves (2 x 2) per CU, each wave holding a 128x128 block of
// fp32 sums (256 accumulation registers) built from v_mfma_f32_16x16x32_bf16.
//
// C[M,N] = sum_k A(m,k) B(k,n); operand orientation as in gemm_bf16.hpp:
//   A_KMAJ: A(m,k) = A[m*lda + k]   else A(m,k) = A[k*lda + m]
//   B_KMAJ: B(k,n) = B[n*ldb + k]   else B(k,n) = B[k*ldb + n]
//
// Why four waves of 128x128 rather than eight of 128x64: every wave reads
// its A and B fragments from LDS once per K step, so the LDS read traffic
// per MFMA falls by a third (a wave reads 128 + 128 rows instead of
// 128 + 64 for half the products).  The one wave per SIMD hides latency by
// software pipelining alone: the fragments of the next 32-deep K substep are
// read while the current substep's 64 MFMAs run, and the global loads of a
// later K step are issued between the first MFMAs of a step.
//
// Data path:
//   * Global -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging); the
//     buffer descriptor is re-based per tile and step, so rows past the end of
//     an operand read as zero.  A K-contiguous tile whose last K step is
//     partial gets its out-of-range chunks zeroed in LDS.
//   * K-contiguous tile: rows of 8 16-byte chunks (K steps of 64), XOR
//     swizzled; one ds_read_b128 gives a lane 8 consecutive K values of one
//     row.  M/N-contiguous tile: 64 K-rows of ROWS elements, XOR swizzled; two
//     ds_read_b64_tr_b16 (gfx950's transposing LDS read) give a lane 8
//     consecutive K values of one column.  Both swizzles (gemm_w4_layout.hpp)
//     keep the fragment reads free of bank conflicts.
//   * Fragment of a 16x32 (rows x K) MFMA operand: lane l holds row l & 15,
//     K values 8 (l >> 4) .. 8 (l >> 4) + 7.  The MFMA takes the B fragment
//     first, so lane l's four sums of a 16x16 block are row l & 15, columns
//     4 (l >> 4) .. 4 (l >> 4) + 3.
//   * Two LDS stages of K steps of 64; the step schedule is described at
//     gemm_w4_body.
//   * Epilogues move the sums to a store layout with lane swaps
//     (permlane16/32_swap, DPP row_ror:8).  fp32 outputs and the saved
//     pre-activation H leave as whole 128-byte lines with non-temporal
//     stores: nothing in the same pass reads them next, and stored that way
//     they leave no dirty lines in L2 or the Infinity Cache for the next
//     kernels to evict.
#pragma once

#include "common.hpp"
#include "gemm.hpp"        // GemmArgs, EpiKind, map_tile
#include "gemm_bf16.hpp"   // pack_bf16x2, bf16lo/hi, waitcnt helpers, lds_char
#include "gemm_w4_layout.hpp"

#include <type_traits>
#include <utility>

namespace tpmlp {

typedef __attribute__((ext_vector_type(4))) float f32x4_w4_t;


// ROWS (M or N) x 64 (K) bf16 operand tile staged by NW waves; NFB fragment
// blocks of 16 rows per wave.
template <int ROWS, bool KMAJ, int NW, int NFB>
struct W4Tile {
  static constexpr int BKT = 64;
  static constexpr int CPR = 8;                // 16-byte chunks per K-contiguous row
  static constexpr int BYTES = ROWS * BKT * 2;
  static constexpr int SLOTS = ROWS * CPR;
  static constexpr int INSTR = SLOTS / (64 * NW);  // buffer loads per wave per step
  static constexpr int QPR = ROWS / 8;         // chunks per K-row (M/N-contiguous)
  static constexpr int NB = KMAJ ? 2 : NFB;    // fragment base registers
  static_assert(SLOTS % (64 * NW) == 0, "tile too small for the waves");
  static_assert(KMAJ || QPR % 8 == 0, "the K-row swizzle works on groups of 8 or 16 chunks");

  uint32_t voff[INSTR];
  uint32_t fbase[NB];

  // w0: the wave's first row (a multiple of 16) in the tile.
  __device__ __forceinline__ void init(int wave, int lane, int64_t ld, int w0) {
#pragma unroll
    for (int j = 0; j < INSTR; ++j) {
      const int s = (wave * INSTR + j) * 64 + lane;
      if constexpr (KMAJ) {
        const int row = s / CPR, c = w4::pos_k(row, s % CPR);   // pos_k is an involution in c
        voff[j] = (uint32_t)(((int64_t)row * ld + c * 8) * 2);
      } else {
        const int k = s / QPR, q = w4::pos_t(QPR, k, s % QPR);  // so is pos_t in q
        voff[j] = (uint32_t)(((int64_t)k * ld + q * 8) * 2);
      }
    }
    if constexpr (KMAJ) {
#pragma unroll
      for (int x = 0; x < NB; ++x) fbase[x] = w4::frag_k_base(w0, lane, x);
    } else {
#pragma unroll
      for (int f = 0; f < NFB; ++f) fbase[f] = w4::frag_t_fast(QPR, w0, lane, f, 0, 0);
    }
  }

  // One of this wave's loads (index j) of one step.  m0 (the LDS address of
  // an LDS-DMA load) is set inside the same asm statement that consumes it;
  // the compiler does not preserve a reserved register listed as clobbered,
  // which is safe because no compiler-generated instruction of these kernels
  // uses m0 (checked on the built library by tests/test_m0_invariant_cpu.py).
  __device__ __forceinline__ void load_one(int j, const i32x4_t& rsrc, lds_char* dst, int wave) const {
    const uint32_t lds = (uint32_t)(uintptr_t)(dst + (wave * INSTR + j) * 1024);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff[j]), "s"(rsrc)
                 : "memory", "m0");
  }

  // K-contiguous tiles: zero this wave's chunks at K offset >= kvalid (the
  // last, partial step; the loads read the next row's data there).
  __device__ __forceinline__ void zero_tail(lds_char* dst, int wave, int lane, int kvalid) const {
    static_assert(KMAJ, "only K-contiguous tiles need the fix-up");
#pragma unroll
    for (int j = 0; j < INSTR; ++j) {
      const int s = (wave * INSTR + j) * 64 + lane;
      const int row = s / CPR, c = w4::pos_k(row, s % CPR);
      if (c * 8 >= kvalid)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(dst + s * 16) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // Fragment block F of substep S: 8 K values of one row (column) per lane.
  template <int F, int S>
  __device__ __forceinline__ u32x4_t frag(const lds_char* src) const {
    if constexpr (KMAJ) {
      return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(src + fbase[S] + F * 2048);
    } else {
      static_assert(F < NFB, "too many fragment blocks");
      const lds_char* p0 = src + fbase[F] + (32 * S) * QPR * 16;
      const lds_char* p1 = p0 + 4 * QPR * 16;
      const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p0);
      const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p1);
      const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0);
      const u32x2_t w1 = __builtin_bit_cast(u32x2_t, v1);
      return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
    }
  }
};

template <int F, int NF, int S>
struct W4FragLoop {
  template <class Tile>
  __device__ __forceinline__ static void run(const Tile& t, const lds_char* src, u32x4_t* out) {
    out[F] = t.template frag<F, S>(src);
    W4FragLoop<F + 1, NF, S>::run(t, src, out);
  }
};
template <int NF, int S>
struct W4FragLoop<NF, NF, S> {
  template <class Tile>
  __device__ __forceinline__ static void run(const Tile&, const lds_char*, u32x4_t*) {}
};

// Calls f(integral_constant<int, I>) for I = 0 .. N-1 in order.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// What follows MFMA t of a substep (in program order): one of NL global loads
// (at t = L0, L0 + LS, ...) and/or one of NR fragment reads (at t = R0,
// R0 + RS, ...).
template <int t, int NL, int L0, int LS, int NR, int R0, int RS>
struct W4Slot {
  static constexpr bool is_load = NL > 0 && t >= L0 && (t - L0) % LS == 0 && (t - L0) / LS < NL;
  static constexpr int load = is_load ? (t - L0) / LS : 0;
  static constexpr bool is_read = NR > 0 && t >= R0 && (t - R0) % RS == 0 && (t - R0) / RS < NR;
  static constexpr int read = is_read ? (t - R0) / RS : 0;
};

// The two LDS stages of a tile size: one array per size, so every
// orientation of a tile size in one kernel (gemm_w4_trio_kernel) shares it.
template <int BYTES>
__device__ __forceinline__ char* w4_lds() {
  __shared__ __attribute__((aligned(1024))) char buf[BYTES];
  return buf;
}

// One workgroup's tile (workgroup pid of the nwg that compute product p).
// K steps of 64 (two 32-deep substeps) through two LDS stages.  Step k:
//   substep 0: MFMAs of (k, 0); reads of (k, 1)'s fragments from stage k.
//   barrier:   this wave's loads of step k + 1 landed; every wave done with
//              stage k (its last fragments were read in substep 0).
//   substep 1: MFMAs of (k, 1); loads of step k + 2 into stage k; reads of
//              (k + 1, 0)'s fragments from stage k + 1.
// So a step's loads have a whole step (128 MFMAs) to land.
// Stores the lane's 16-byte values v0, v1 of block pairs jj0 and jj0 + 1 of a
// 16-row block (8 consecutive bf16 of row (lane & 15) from column
// 32 jj + coff, the store layout of the epilogues) as whole 128-byte lines:
// the lanes of rows 8-15 of each 16-lane row swap with those of rows 0-7 (DPP
// row_ror:8), so one store covers rows 0-7 and one rows 8-15, each row's 64
// columns from 8 lanes.  row0, col0: the block's first row and pair jj0's
// first column (col0 a multiple of 64, so the lines are whole).
template <bool NT>
__device__ __forceinline__ void w4_store_pair_lines(bf16_t* base, int64_t ld, int row0, int col0, int M, int N,
                                                    int lane, int coff, const u32x4_t& v0, const u32x4_t& v1) {
  const bool lower = (lane & 15) < 8;
  u32x4_t a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)(lower ? v1[e] : v0[e]), 0x128, 0xf, 0xf, false);
    a[e] = lower ? v0[e] : r;
    b[e] = lower ? r : v1[e];
  }
  const int rowA = row0 + (lane & 7), rowB = rowA + 8;
  const int cs = col0 + (lower ? 0 : 32) + coff;
  if (cs >= N) return;
  if (rowA < M) {
    u32x4_t* d = reinterpret_cast<u32x4_t*>(base + (int64_t)rowA * ld + cs);
    if constexpr (NT) __builtin_nontemporal_store(a, d);
    else *d = a;
  }
  if (rowB < M) {
    u32x4_t* d = reinterpret_cast<u32x4_t*>(base + (int64_t)rowB * ld + cs);
    if constexpr (NT) __builtin_nontemporal_store(b, d);
    else *d = b;
  }
}

// The lane's 16-byte value of one block pair in the store layout, as a plain
// store (the two halves of a line from neighbouring pairs meet in L2).
__device__ __forceinline__ void w4_store_pair(bf16_t* base, int64_t ld, int row, int cs, int M, int N,
                                              const u32x4_t& v) {
  if (row < M && cs < N) *reinterpret_cast<u32x4_t*>(base + (int64_t)row * ld + cs) = v;
}

template <int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI>
__device__ __forceinline__ void gemm_w4_body(const GemmArgs& p, int pid, int nwg) {
  constexpr int WGM = 2, WGN = 2, NW = 4, NT = 256, BKT = 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of whole pairs of 16-row blocks");
  using TA = W4Tile<BM, A_KMAJ, NW, FM>;
  using TB = W4Tile<BN, B_KMAJ, NW, FN>;
  constexpr int STAGE = TA::BYTES + TB::BYTES;
  constexpr int LPS = TA::INSTR + TB::INSTR;  // buffer loads per wave per step
  static_assert(2 * STAGE <= 160 * 1024, "LDS");

  char* const st0 = w4_lds<2 * STAGE>();
  char* const st1 = st0 + STAGE;
  auto stage = [&](auto I) -> lds_char* {
    if constexpr (decltype(I)::value == 0) return (lds_char*)st0;
    else return (lds_char*)st1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

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
  const int nkp = (nk + 1) & ~1;                 // the loop body is two steps
  const int ktail = (kend - kbeg) & (BKT - 1);   // valid K in the last step (0: full)

  const bf16_t* A = static_cast<const bf16_t*>(p.A);
  const bf16_t* B = static_cast<const bf16_t*>(p.B);
  TA ta;
  TB tb;
  ta.init(wave, lane, p.lda, wm * WTM);
  tb.init(wave, lane, p.ldb, wn * WTN);

  // Buffer descriptors of step kt: base + kt * stride, and the byte count
  // past which loads read zero (rows past the operand, K past its end).  A
  // step past the end of K gets an empty descriptor: its loads write zeros,
  // so every step issues the same loads and the loop has no branch.
  struct StepDesc {
    uint64_t base0;       // byte address of step 0
    uint64_t stride;      // bytes between steps
    uint32_t nb0, dnb;    // byte count of step kt: nb0 - kt * dnb (K-contiguous) ...
    uint32_t nb_last;     // ... or nb0 for full steps and nb_last for the last (M/N-contiguous)
  };
  auto make_desc = [&](const bf16_t* X, int64_t ld, int r0, int R, int TR, bool kmaj) {
    StepDesc d;
    if (kmaj) {
      const int rows = min(TR, R - r0);
      d.base0 = reinterpret_cast<uint64_t>(X + (int64_t)r0 * ld + kbeg);
      d.stride = BKT * 2;
      d.nb0 = (uint32_t)(((int64_t)(rows - 1) * ld + (kend - kbeg)) * 2);
      d.dnb = BKT * 2;
      d.nb_last = 0;
    } else {
      const int kv_last = (kend - kbeg) - (nk - 1) * BKT;
      d.base0 = reinterpret_cast<uint64_t>(X + (int64_t)kbeg * ld + r0);
      d.stride = (uint64_t)BKT * ld * 2;
      d.nb0 = (uint32_t)(((int64_t)(BKT - 1) * ld + (R - r0)) * 2);
      d.dnb = 0;
      d.nb_last = (uint32_t)(((int64_t)(kv_last - 1) * ld + (R - r0)) * 2);
    }
    return d;
  };
  const StepDesc da = make_desc(A, p.lda, m0, M, BM, A_KMAJ);
  const StepDesc db = make_desc(B, p.ldb, n0, N, BN, B_KMAJ);
  auto rsrc_step = [&](const StepDesc& d, bool kmaj, int kt) {
    const uint64_t addr = d.base0 + (uint64_t)kt * d.stride;
    uint32_t nb = kmaj ? d.nb0 - (uint32_t)kt * d.dnb : (kt == nk - 1 ? d.nb_last : d.nb0);
    nb = kt < nk ? nb : 0u;
    return i32x4_t{(int)(uint32_t)addr, (int)((addr >> 32) & 0xffffu), (int)nb, kBufferWord3};
  };
  auto rsrc_a = [&](int kt) { return rsrc_step(da, A_KMAJ, kt); };
  auto rsrc_b = [&](int kt) { return rsrc_step(db, B_KMAJ, kt); };
  auto issue = [&](int kt, lds_char* dst) {
    const i32x4_t ra = rsrc_a(kt), rb = rsrc_b(kt);
#pragma unroll
    for (int j = 0; j < TA::INSTR; ++j) ta.load_one(j, ra, dst, wave);
#pragma unroll
    for (int j = 0; j < TB::INSTR; ++j) tb.load_one(j, rb, dst + TA::BYTES, wave);
  };
  const int tail_kt = ktail != 0 ? nk - 1 : -2;   // the partial last step, if any
  auto fix_tail = [&](int kt, lds_char* dst) {
    if (kt == tail_kt) {
      if constexpr (A_KMAJ) ta.zero_tail(dst, wave, lane, ktail);
      if constexpr (B_KMAJ) tb.zero_tail(dst + TA::BYTES, wave, lane, ktail);
    }
  };
  // Before the barrier: this wave's loads of step kt_next landed (LATER
  // steps' loads may still be in flight), its zero writes and fragment reads
  // done.
  auto sync = [&](int kt_next, lds_char* dst, auto LATER) {
    constexpr int later = decltype(LATER)::value;
    static_assert(later * LPS < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(later * LPS));
    fix_tail(kt_next, dst);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
  };

  // The sums live in AGPRs: the MFMAs are inline asm with "+a" operands
  // (the compiler's own choice of VGPR sums spilled heavily at this size).
  f32x4_w4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      acc[i][j] = f32x4_w4_t{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[i][j]));
    }

  u32x4_t fa[2][FM], fb[2][FN];  // fragments of the two substeps

  // Fragment read number t of a substep into buffer D, in the order the
  // MFMAs use them: A block 0, the B blocks, then the other A blocks.
  constexpr int NFRAG = FM + FN;
  auto read_frag = [&](auto TC, auto SC, auto DC, const lds_char* src) {
    constexpr int t = decltype(TC)::value, S = decltype(SC)::value, D = decltype(DC)::value;
    if constexpr (t == 0) fa[D][0] = ta.template frag<0, S>(src);
    else if constexpr (t <= FN) fb[D][t - 1] = tb.template frag<(t - 1 < FN ? t - 1 : 0), S>(src + TA::BYTES);
    else fa[D][t - FN] = ta.template frag<(t - FN < FM ? t - FN : 0), S>(src);
  };
  // Descriptors of the loads the next substep 1 issues, formed between the
  // MFMAs of substep 0 (scalar work kept out of the load stretch).
  i32x4_t ld_ra = {0, 0, 0, 0}, ld_rb = {0, 0, 0, 0};
  // The FM x FN MFMAs of buffer D in program order; after MFMA t, the slot's
  // global load (step `lkt`'s descriptors in ld_ra/ld_rb, into `ldst`)
  // and/or fragment read (substep S2 into buffer D2, from `rsrc`); a
  // scheduling barrier pins the order.
  constexpr int kDescAt = FM * FN / 2;   // substep 0 forms the next descriptors after this MFMA
  auto substep = [&](auto DC, auto NLC, auto L0C, auto LSC, auto R0C, auto RSC, auto S2C, auto D2C,
                     auto DESC, int dkt, lds_char* ldst, const lds_char* rsrc) {
    constexpr int D = decltype(DC)::value, NL = decltype(NLC)::value, L0 = decltype(L0C)::value,
                  LS = decltype(LSC)::value, R0 = decltype(R0C)::value, RS = decltype(RSC)::value;
    static_for<FM * FN>([&](auto TC) {
      constexpr int t = decltype(TC)::value;
      constexpr int i = t / FN, j = t % FN;
      using SL = W4Slot<t, NL, L0, LS, NFRAG, R0, RS>;
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fb[D][j]), "v"(fa[D][i]));
      if constexpr (SL::is_load) {
        if constexpr (SL::load < TA::INSTR) ta.load_one(SL::load, ld_ra, ldst, wave);
        else tb.load_one(SL::load - TA::INSTR, ld_rb, ldst + TA::BYTES, wave);
      }
      if constexpr (SL::is_read) read_frag(std::integral_constant<int, SL::read>{}, S2C, D2C, rsrc);
      // (the empty asm pins the scalar work here, between the MFMAs)
      if constexpr (decltype(DESC)::value && t == kDescAt) {
        ld_ra = rsrc_a(dkt);
        asm volatile("" : "+s"(ld_ra));
      }
      if constexpr (decltype(DESC)::value && t == kDescAt + 4) {
        ld_rb = rsrc_b(dkt);
        asm volatile("" : "+s"(ld_rb));
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // Slot patterns: substep 0 reads one fragment after each of its first
  // MFMAs; substep 1 reads one after each odd MFMA of its first half and
  // spreads its global loads evenly over all of its MFMAs (a burst of loads
  // fills the texture-address queue, and the in-order wave then stalls its
  // MFMAs behind a load).
  constexpr int kLoadStride = FM * FN / LPS;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  static_assert(kLoadStride >= 2 && 2 * NFRAG <= FM * FN, "loads and reads fit between the MFMAs");

  auto step = [&](auto STc, int kt) {
    constexpr int ST = decltype(STc)::value;
    lds_char* cur = stage(STc);
    lds_char* nxt = stage(std::integral_constant<int, 1 - ST>{});
    substep(I0{}, I0{}, I0{}, I1{}, I0{}, I1{}, I1{}, I1{}, std::true_type{}, kt + 2, nullptr, cur);
    sync(kt + 1, nxt, I0{});
    substep(I1{}, std::integral_constant<int, LPS>{}, I0{}, std::integral_constant<int, kLoadStride>{}, I1{}, I2{}, I0{}, I0{}, std::false_type{}, 0,
            cur, nxt);
  };

  if (nk > 0) {
    issue(0, stage(I0{}));
    issue(1, stage(I1{}));
    sync(0, stage(I0{}), I1{});
    static_for<NFRAG>([&](auto TC) { read_frag(TC, I0{}, I0{}, stage(I0{})); });
    for (int kt = 0; kt < nkp; kt += 2) {
      step(I0{}, kt);
      step(I1{}, kt + 1);
    }
  }
  // The inline-asm MFMAs are invisible to the compiler's hazard tracking:
  // wait out the longest MFMA-write -> VALU/VMEM-read distance before the
  // epilogue reads the sums.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // Epilogues take the sums one row block at a time: a scheduling fence and
  // an empty asm that redefines the block's AGPRs keep the compiler from
  // copying all 256 sums to VGPRs at once (which spills).
  auto row_block = [&](int i) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
  };
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // drain the loads the compiler does not see
  __syncthreads();
  if (p.clk != nullptr && pid == 0 && tid == 0) {
    p.clk[0] = __builtin_amdgcn_s_memtime() - clk0;
    p.clk[1] = __builtin_amdgcn_s_memrealtime() - ref0;
  }
  float* red = reinterpret_cast<float*>(st0);  // epilogue scratch (LDS is free now)
  (void)red;

  // ------------------------------------------------------------ epilogue --
  // Lane l, block (i, j), register v: row m0 + wm*WTM + 16 i + (l & 15),
  // column n0 + wn*WTN + 16 j + 4 (l >> 4) + v.
  const int g4 = lane >> 4;
  const int mrow = m0 + wm * WTM + (lane & 15);
  const int ncol = n0 + wn * WTN + 4 * g4;
  // After permlane16_swap of blocks (2jj, 2jj+1) lane group g holds 8
  // consecutive columns starting at 32 jj + coff of the wave's columns.
  const int coff = 16 * (g4 & 1) + 8 * (g4 >> 1);
  if constexpr (EPI == kEpiF32) {
    float* __restrict__ C = p.C + (int64_t)ks * p.split_stride;
    // Non-temporal stores of whole 128-byte lines: for blocks (2jj, 2jj+1)
    // the lanes of rows 8-15 of a 16-lane row swap with those of rows 0-7
    // (DPP row_ror:8), so one store covers rows 0-7 and one rows 8-15, each
    // row's 32 columns from 8 lanes.
    const bool lower = (lane & 15) < 8;
    const int rsub = lane & 7;
    const int csub = 4 * g4 + (lower ? 0 : 16);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      row_block(i);
      const int rowA = m0 + wm * WTM + 16 * i + rsub, rowB = rowA + 8;
#pragma unroll
      for (int jj = 0; jj < FN / 2; ++jj) {
        const int col = n0 + wn * WTN + 32 * jj + csub;
        f32x4_w4_t a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[i][2 * jj][e], y = acc[i][2 * jj + 1][e];
          const float r = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(lower ? y : x), 0x128, 0xf, 0xf, false));
          a[e] = lower ? x : r;
          b[e] = lower ? r : y;
        }
        if (col < N) {
          if (rowA < M) __builtin_nontemporal_store(a, reinterpret_cast<f32x4_w4_t*>(C + (int64_t)rowA * p.ldc + col));
          if (rowB < M) __builtin_nontemporal_store(b, reinterpret_cast<f32x4_w4_t*>(C + (int64_t)rowB * p.ldc + col));
        }
      }
    }
  } else if constexpr (EPI == kEpiBiasAct) {
    auto epilogue = [&](auto GeluC) {
      constexpr bool kGelu = decltype(GeluC)::value;
      bf16_t* __restrict__ Y = static_cast<bf16_t*>(p.Y);
      bf16_t* __restrict__ Hs = static_cast<bf16_t*>(p.H);
      const bf16_t* __restrict__ bias = static_cast<const bf16_t*>(p.bias);
      // bias of the lane's columns (4 per block), loaded together before use
      u32x2_t bw[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int c = ncol + 16 * j;
        bw[j] = u32x2_t{0u, 0u};
        if (bias && c < N) bw[j] = *reinterpret_cast<const u32x2_t*>(bias + c);
      }
      // A and H of block pair jj in the store layout: 8 consecutive columns
      // from 32 jj + coff (a permlane16_swap of the pair's packed values).
      auto pair_values = [&](int i, int jj, u32x4_t& av, u32x4_t& hvv) {
        uint32_t aw[2][2], hw[2][2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int j = 2 * jj + q;
          const float hv[4] = {acc[i][j][0] + bf16lo(bw[j][0]), acc[i][j][1] + bf16hi(bw[j][0]),
                               acc[i][j][2] + bf16lo(bw[j][1]), acc[i][j][3] + bf16hi(bw[j][1])};
          if constexpr (kGelu) {
            aw[q][0] = pack_bf16x2(gelu_tanh(hv[0]), gelu_tanh(hv[1]));
            aw[q][1] = pack_bf16x2(gelu_tanh(hv[2]), gelu_tanh(hv[3]));
          } else {
            aw[q][0] = pack_bf16x2(hv[0], hv[1]);
            aw[q][1] = pack_bf16x2(hv[2], hv[3]);
          }
          hw[q][0] = pack_bf16x2(hv[0], hv[1]);
          hw[q][1] = pack_bf16x2(hv[2], hv[3]);
        }
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const auto ra = __builtin_amdgcn_permlane16_swap(aw[0][w], aw[1][w], false, false);
          aw[0][w] = ra[0];
          aw[1][w] = ra[1];
          const auto rh = __builtin_amdgcn_permlane16_swap(hw[0][w], hw[1][w], false, false);
          hw[0][w] = rh[0];
          hw[1][w] = rh[1];
        }
        av = u32x4_t{aw[0][0], aw[0][1], aw[1][0], aw[1][1]};
        hvv = u32x4_t{hw[0][0], hw[0][1], hw[1][0], hw[1][1]};
      };
      // A (read by the next product) as plain stores, H (kept for the
      // backward pass) as non-temporal ones; both in whole lines where the
      // wave's columns allow: pairs (0,1), (2,3) at 256x256 and 128x128; at
      // 256x192 (three pairs, 96 columns a wave) pairs (0,1) of wave column 0
      // and (1,2) of wave column 1, the pair between them (one line shared
      // by the two waves) as plain half-line stores.
      auto two = [&](int i, int jj0) {
        u32x4_t a0, h0, a1, h1;
        pair_values(i, jj0, a0, h0);
        pair_values(i, jj0 + 1, a1, h1);
        const int row0 = m0 + wm * WTM + 16 * i, col0 = n0 + wn * WTN + 32 * jj0;
        w4_store_pair_lines<false>(Y, p.ldy, row0, col0, M, N, lane, coff, a0, a1);
        if (Hs) w4_store_pair_lines<true>(Hs, p.ldh, row0, col0, M, N, lane, coff, h0, h1);
      };
      auto one = [&](int i, int jj) {
        u32x4_t av, hv;
        pair_values(i, jj, av, hv);
        const int row = mrow + 16 * i, cs = n0 + wn * WTN + 32 * jj + coff;
        w4_store_pair(Y, p.ldy, row, cs, M, N, av);
        if (Hs) w4_store_pair(Hs, p.ldh, row, cs, M, N, hv);
      };
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        row_block(i);
        if constexpr ((FN / 2) % 2 == 0) {
#pragma unroll
          for (int jp = 0; jp < FN / 4; ++jp) two(i, 2 * jp);
        } else {
          static_assert(FN / 2 == 3, "three block pairs a wave (256x192) when not even");
          if (wn == 0) {
            two(i, 0);
            one(i, 2);
          } else {
            one(i, 0);
            two(i, 1);
          }
        }
      }
    };
    if (p.act == kActGeluTanh) epilogue(std::true_type{});
    else epilogue(std::false_type{});
  } else if constexpr (EPI == kEpiActBwd) {
    // Lanes take their sums to the store layout first (a permlane16_swap of
    // the fp32 values of block pair (2jj, 2jj+1): 8 consecutive columns from
    // 32 jj + coff), so H is read as one 16-byte load per block pair.
    auto epilogue = [&](auto GeluC) {
      constexpr bool kGelu = decltype(GeluC)::value;
      bf16_t* __restrict__ Y = static_cast<bf16_t*>(p.Y);
      const bf16_t* __restrict__ Hs = static_cast<const bf16_t*>(p.H);
      float csum[FN / 2][8];
#pragma unroll
      for (int jj = 0; jj < FN / 2; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e) csum[jj][e] = 0.f;
      // H of row block i goes out two blocks ahead of its use.
      u32x4_t hq[FM][FN / 2];
      auto load_h = [&](int i) {
#pragma unroll
        for (int jj = 0; jj < FN / 2; ++jj) {
          hq[i][jj] = u32x4_t{0u, 0u, 0u, 0u};
          if constexpr (kGelu) {
            const int row = mrow + 16 * i, cs = n0 + wn * WTN + 32 * jj + coff;
            if (row < M && cs < N) hq[i][jj] = *reinterpret_cast<const u32x4_t*>(Hs + (int64_t)row * p.ldh + cs);
          }
        }
      };
      load_h(0);
      if constexpr (FM > 1) load_h(1);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        row_block(i);
        if (i + 2 < FM) load_h(i + 2);
        const int row = mrow + 16 * i;
#pragma unroll
        for (int jj = 0; jj < FN / 2; ++jj) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][2 * jj][e]),
                                                            __float_as_uint(acc[i][2 * jj + 1][e]), false, false);
            x[e] = __uint_as_float(r[0]);
            x[4 + e] = __uint_as_float(r[1]);
          }
          const int cs = n0 + wn * WTN + 32 * jj + coff;
          float d[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) d[e] = 0.f;
          if (row < M && cs < N) {
            if constexpr (kGelu) {
              const u32x4_t hw = hq[i][jj];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float hv = (e & 1) ? bf16hi(hw[e >> 1]) : bf16lo(hw[e >> 1]);
                d[e] = x[e] * gelu_tanh_grad(hv);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) d[e] = x[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) csum[jj][e] += d[e];
            *reinterpret_cast<u32x4_t*>(Y + (int64_t)row * p.ldy + cs) =
                u32x4_t{pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]), pack_bf16x2(d[4], d[5]), pack_bf16x2(d[6], d[7])};
          }
        }
      }
      if (p.colsum) {
#pragma unroll
        for (int jj = 0; jj < FN / 2; ++jj)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
#pragma unroll
            for (int x = 1; x < 16; x <<= 1) csum[jj][e] += __shfl_xor(csum[jj][e], x);
          }
        if ((lane & 15) == 0) {
#pragma unroll
          for (int jj = 0; jj < FN / 2; ++jj)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wm * BN + wn * WTN + 32 * jj + coff + e] = csum[jj][e];
        }
      }
    };
    if (p.act == kActGeluTanh) epilogue(std::true_type{});
    else epilogue(std::false_type{});
    if (p.colsum) {
      __syncthreads();
      for (int c = tid; c < BN; c += NT) {
        const float t = red[c] + red[BN + c];   // wave rows in order
        if (n0 + c < N) p.colsum[(int64_t)tmi * N + n0 + c] = t;
      }
    }
  } else if constexpr (EPI == kEpiSwiGLU) {
    // Packed column 16q + r holds gate (r < 8) or up (r >= 8) of output
    // column 8q + r % 8: block j of 16 packed columns is one q, whose gate
    // values sit in lane groups 0, 1 and up values in groups 2, 3.  A
    // permlane32_swap of blocks (2jj, 2jj+1) gives lanes 0-31 gate and up of
    // block 2jj and lanes 32-63 those of block 2jj+1, each lane 4 output
    // columns.
    bf16_t* __restrict__ Y = static_cast<bf16_t*>(p.Y);   // [M, N/2]
    bf16_t* __restrict__ Hs = static_cast<bf16_t*>(p.H);  // [M, N] packed, or null
    // Block pair jj of row block i: stores silu(gate) * up (8 bytes a lane,
    // plain: the next product reads it) and returns the packed gate/up
    // values in the store layout (8 consecutive packed columns from
    // 32 jj + coff).
    auto pair_a = [&](int i, int jj) -> u32x4_t {
      const int j0 = 2 * jj;
      uint32_t hw[2][2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        hw[q][0] = pack_bf16x2(acc[i][j0 + q][0], acc[i][j0 + q][1]);
        hw[q][1] = pack_bf16x2(acc[i][j0 + q][2], acc[i][j0 + q][3]);
      }
      float gv[4], uv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j0][e]),
                                                        __float_as_uint(acc[i][j0 + 1][e]), false, false);
        gv[e] = __uint_as_float(r[0]);
        uv[e] = __uint_as_float(r[1]);
      }
      uint32_t aw[2];
      {
        float av[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = gv[e] * sigmoidf_fast(gv[e]) * uv[e];
        aw[0] = pack_bf16x2(av[0], av[1]);
        aw[1] = pack_bf16x2(av[2], av[3]);
      }
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const auto rh = __builtin_amdgcn_permlane16_swap(hw[0][w], hw[1][w], false, false);
        hw[0][w] = rh[0];
        hw[1][w] = rh[1];
      }
      const int row = mrow + 16 * i;
      // lanes 0-31: block 2jj, lanes 32-63: block 2jj+1; group parity picks r 0..3 or 4..7
      const int pc = n0 + wn * WTN + 16 * (j0 + (g4 >> 1));   // packed column of the block, 16q
      if (row < M && pc < N)
        *reinterpret_cast<u32x2_t*>(Y + (int64_t)row * p.ldy + pc / 2 + 4 * (g4 & 1)) = u32x2_t{aw[0], aw[1]};
      return u32x4_t{hw[0][0], hw[0][1], hw[1][0], hw[1][1]};
    };
    // gate/up, kept for the backward pass, as whole lines with non-temporal
    // stores where the wave's columns allow (as H in the bias+GeLU epilogue).
    auto two = [&](int i, int jj0) {
      const u32x4_t g0 = pair_a(i, jj0), g1 = pair_a(i, jj0 + 1);
      if (Hs)
        w4_store_pair_lines<true>(Hs, p.ldh, m0 + wm * WTM + 16 * i, n0 + wn * WTN + 32 * jj0, M, N, lane, coff, g0,
                                  g1);
    };
    auto one = [&](int i, int jj) {
      const u32x4_t g = pair_a(i, jj);
      if (Hs) w4_store_pair(Hs, p.ldh, mrow + 16 * i, n0 + wn * WTN + 32 * jj + coff, M, N, g);
    };
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      row_block(i);
      if constexpr ((FN / 2) % 2 == 0) {
#pragma unroll
        for (int jp = 0; jp < FN / 4; ++jp) two(i, 2 * jp);
      } else {
        static_assert(FN / 2 == 3, "three block pairs a wave (256x192) when not even");
        if (wn == 0) {
          two(i, 0);
          one(i, 2);
        } else {
          one(i, 0);
          two(i, 1);
        }
      }
    }
  } else {  // kEpiSwiGLUBwd
    // acc = dA for output columns c (N of them).  Column c = 8q + r reads gate
    // and up at packed columns 16q + r and 16q + 8 + r of H and writes dgate
    // and dup to the same packed columns of Y.  Lanes take their sums to the
    // store layout first (a permlane16_swap of the fp32 values of block pair
    // (2jj, 2jj+1)): 8 consecutive columns from c0 = 32 jj + coff, one whole
    // q, so gate, up, dgate and dup each move as one 16-byte access.
    bf16_t* __restrict__ Y = static_cast<bf16_t*>(p.Y);               // [M, 2N] packed
    const bf16_t* __restrict__ Hs = static_cast<const bf16_t*>(p.H);  // [M, 2N] packed
    // gate and up of row block i go out one block ahead of their use
    u32x4_t gq[FM][FN / 2], uq[FM][FN / 2];
    auto load_gu = [&](int i) {
#pragma unroll
      for (int jj = 0; jj < FN / 2; ++jj) {
        const int row = mrow + 16 * i, c0 = n0 + wn * WTN + 32 * jj + coff;
        gq[i][jj] = uq[i][jj] = u32x4_t{0u, 0u, 0u, 0u};
        if (row < M && c0 < N) {
          const bf16_t* src = Hs + (int64_t)row * p.ldh + 2 * c0;
          gq[i][jj] = *reinterpret_cast<const u32x4_t*>(src);
          uq[i][jj] = *reinterpret_cast<const u32x4_t*>(src + 8);
        }
      }
    };
    load_gu(0);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      row_block(i);
      if (i + 1 < FM) load_gu(i + 1);
      const int row = mrow + 16 * i;
#pragma unroll
      for (int jj = 0; jj < FN / 2; ++jj) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][2 * jj][e]),
                                                          __float_as_uint(acc[i][2 * jj + 1][e]), false, false);
          x[e] = __uint_as_float(r[0]);
          x[4 + e] = __uint_as_float(r[1]);
        }
        const int c0 = n0 + wn * WTN + 32 * jj + coff;
        if (row < M && c0 < N) {
          uint32_t dgw[4], duw[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            float dg[2], du[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float gv = h ? bf16hi(gq[i][jj][w]) : bf16lo(gq[i][jj][w]);
              const float uv = h ? bf16hi(uq[i][jj][w]) : bf16lo(uq[i][jj][w]);
              float sl, sg;
              silu_and_grad(gv, sl, sg);
              dg[h] = x[2 * w + h] * uv * sg;
              du[h] = x[2 * w + h] * sl;
            }
            dgw[w] = pack_bf16x2(dg[0], dg[1]);
            duw[w] = pack_bf16x2(du[0], du[1]);
          }
          bf16_t* dst = Y + (int64_t)row * p.ldy + 2 * c0;
          *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{dgw[0], dgw[1], dgw[2], dgw[3]};
          *reinterpret_cast<u32x4_t*>(dst + 8) = u32x4_t{duw[0], duw[1], duw[2], duw[3]};
        }
      }
    }
  }
}

template <int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ void __launch_bounds__(256, 1) gemm_w4_kernel(const GemmArgs p) {
  gemm_w4_body<BM, BN, A_KMAJ, B_KMAJ, EPI>(p, (int)blockIdx.x, (int)gridDim.x);
}

// Two independent products in one launch: workgroups [0, n0) compute p0, the
// rest p1 (n0 a multiple of 8, so each workgroup keeps its XCD).
template <int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ void __launch_bounds__(256, 1) gemm_w4_pair_kernel(const GemmArgs p0, const GemmArgs p1, int n0) {
  if ((int)blockIdx.x < n0)
    gemm_w4_body<BM, BN, A_KMAJ, B_KMAJ, EPI>(p0, (int)blockIdx.x, n0);
  else
    gemm_w4_body<BM, BN, A_KMAJ, B_KMAJ, EPI>(p1, (int)blockIdx.x - n0, (int)gridDim.x - n0);
}

// Two independent products with different operand layouts or epilogues in
// one launch: workgroups [0, n0) compute p0 and are dispatched first, the rest
// p1 (n0 a multiple of 8, so each workgroup keeps its XCD within its product).
// With p0 the product of longer tiles, p1's tiles fill the CUs that p0's
// leave free and then the CUs its tiles release.
template <int BM, int BN, bool AK0, bool BK0, int E0, bool AK1, bool BK1, int E1>
__global__ void __launch_bounds__(256, 1) gemm_w4_duo_kernel(const GemmArgs p0, const GemmArgs p1, int n0) {
  if ((int)blockIdx.x < n0)
    gemm_w4_body<BM, BN, AK0, BK0, E0>(p0, (int)blockIdx.x, n0);
  else
    gemm_w4_body<BM, BN, AK1, BK1, E1>(p1, (int)blockIdx.x - n0, (int)gridDim.x - n0);
}

// The MLP backward's two weight gradients (both operands M/N-contiguous) and
// its input gradient (both K-contiguous), independent of each other, in one
// launch: workgroups [0, n0) compute p0, [n0, n0 + n1) p1, the rest p2 (n0
// and n1 multiples of 8, so each workgroup keeps its XCD within its product).
template <int BM, int BN>
__global__ void __launch_bounds__(256, 1)
gemm_w4_trio_kernel(const GemmArgs p0, const GemmArgs p1, const GemmArgs p2, int n0, int n1) {
  const int b = (int)blockIdx.x;
  if (b < n0)
    gemm_w4_body<BM, BN, false, false, kEpiF32>(p0, b, n0);
  else if (b < n0 + n1)
    gemm_w4_body<BM, BN, false, false, kEpiF32>(p1, b - n0, n1);
  else
    gemm_w4_body<BM, BN, true, true, kEpiF32>(p2, b - n0 - n1, (int)gridDim.x - n0 - n1);
}

}  // namespace tpmlp
