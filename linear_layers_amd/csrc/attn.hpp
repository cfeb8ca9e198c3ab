// Attention core of one shard's heads on gfx950: O = softmax(Q K^T * scale) V
// per head and sequence (optional causal mask), computed flash-style: a
// workgroup owns 128 query rows of one head, streams the keys and values in
// blocks of 64 through LDS and keeps a running row maximum and sum (the
// online softmax of sunjinbo.space/document/parallelism.html, CP · 上下文并行:
// a query block's attention accumulated key block by key block).  Heads are
// independent (damodev.csdn.net/6a43867610ee7a33f284fb9e.html, 1.2.2; the
// head-sharded projections on io.zouht.com/197.html, 2.2.1), so the grid is
// (work items, heads, batch).  When causal, a query block's keys are cut into
// chunks (one workgroup each) so that no workgroup's share is much longer than
// another's and the grid holds enough workgroups to fill the chip; the
// normalised partial results of a block's chunks are merged by their
// log-sum-exp (attn_fwd_combine_kernel).
//
// Layout: T = batch * seq token rows; head h reads columns [128h, 128h+128)
// of Q, K and V (each with its own row stride, e.g. the three blocks of the
// fused QKV projection output) and writes the same columns of O.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, B fragment first as in the GEMM):
//   S = Q K^T: a wave's 32 query rows are the A fragments (held in registers
//     for all 8 K-substeps of head_dim 128); K is a K-contiguous tile (64 keys
//     x 64 of d, two per block) read with ds_read_b128.
//   O += P V: P (bf16) is the A operand; V is an M/N-contiguous tile (64 key
//     rows x 128 of d) read with ds_read_b64_tr_b16.
//   A lane holds row (lane & 31) of S with 4-column groups; a lane-pair swap
//   (v_permlane32_swap) turns those groups into the 8 consecutive keys an A
//   fragment needs, the same exchange the GEMM epilogues use for stores.
#pragma once

#include <utility>

#include "gemm_bf16.hpp"

namespace tpmlp {

struct AttnArgs {
  const bf16_t* Q;
  const bf16_t* K;
  const bf16_t* V;
  int64_t ldq, ldk, ldv;
  bf16_t* O;
  int64_t ldo;
  float* lse;         // [heads, batch * seq] natural-log row log-sum-exp, or null
  int batch, seq, heads, causal;
  float scale_log2;   // scale * log2(e): scores are kept in base-2 units
  // causal key chunks (see attn_key_chunks); partials of blocks with several
  float* o_part;      // [batch][heads][items][128][128] fp32 O of one chunk, normalised by its own sum
  float* lse_part;    // [batch][heads][items][128] base-2 log-sum-exp of that chunk
  int chunks, kc, items;
};

constexpr int kAttnD = 128;   // head_dim
constexpr int kAttnBQ = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kAttnBK = 64;   // keys per block

// Causal work split along keys: query block b of 128 rows sees up to 2 (b + 1)
// key blocks of 64; they are taken in chunks of kc key blocks (kc even: 26,
// more where a block would otherwise have more than 8 chunks), one workgroup
// per (block, chunk).  Chunk c exists for blocks b >= c * kc / 2.  Work items are numbered
// chunk by chunk, the blocks of one chunk from the last down:
// item(b, c) = sum over c' < c of (nqb - c' kc / 2), plus nqb - 1 - b.
__device__ __forceinline__ int attn_key_chunks(int b, int seq, int kc) {
  const int kv_end = min(seq, (b + 1) * 128);
  return ((kv_end + 63) / 64 + kc - 1) / kc;
}
using AttnKTile = Bf16Tile<kAttnBK, true, 64, 4>;   // 64 keys x 64 of d, K-contiguous
using AttnVTile = Bf16Tile<kAttnD, false, 64, 4>;   // 64 key rows x 128 of d, d contiguous
constexpr int kAttnStage = 2 * AttnKTile::BYTES + AttnVTile::BYTES;  // 32 KB

__device__ __forceinline__ f32x16_t mfma_bf16(const u32x4_t& b, const u32x4_t& a, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b), __builtin_bit_cast(bf16x8_t, a),
                                                  c, 0, 0, 0);
}

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// The same product with the accumulator pinned to accumulation registers
// (AGPRs) for long-lived sums.  The compiler does not see into the asm, so it
// covers the hazards itself: NOP_A wait states before the product when `a`
// may just have been written by a VALU op (which needs 2), and
// agpr_acc_drain before any VALU read of the sums (the product's passes + 2).
template <int NOP_A>
__device__ __forceinline__ void mfma_bf16_agpr(const u32x4_t& b, const u32x4_t& a, f32x16_t& c) {
  if constexpr (NOP_A > 0)
    asm volatile("s_nop %3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a), "n"(NOP_A - 1));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
}

// 24 wait states after the last product into any of the sums, ordered before
// every later use of them.
__device__ __forceinline__ void agpr_acc_drain(f32x16_t (&x)[4], f32x16_t (&y)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(y[0]), "+a"(y[1]), "+a"(y[2]), "+a"(y[3]));
}
__device__ __forceinline__ void agpr_acc_drain(f32x16_t (&x)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]));
}

// Lane-pair exchange of two register groups g0 = (x0, x1) and g1 = (y0, y1),
// each 4 bf16 of columns 4h..4h+3 of their 8-column group: afterwards lane
// h = 0 holds the 8 columns of g0 and lane h = 1 those of g1, as
// {x0, x1, y0, y1}.
__device__ __forceinline__ u32x4_t swap_pack(uint32_t x0, uint32_t x1, uint32_t y0, uint32_t y1) {
  const auto r0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
  const auto r1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
  return u32x4_t{r0[0], r1[0], r0[1], r1[1]};
}

// S for one block: 8 K-substeps of 16 over head_dim, two 32-key fragments.
template <int SS>
__device__ __forceinline__ void attn_qk_step(const AttnKTile& kt, const lds_char* kst, const u32x4_t (&qf)[8],
                                             f32x16_t (&s)[2]) {
  u32x4_t kb[2];
  FragLoop<0, 2, SS % 4>::run(kt, kst + (SS / 4) * AttnKTile::BYTES, kb);
  s[0] = mfma_bf16(kb[0], qf[SS], s[0]);
  s[1] = mfma_bf16(kb[1], qf[SS], s[1]);
  if constexpr (SS + 1 < 8) attn_qk_step<SS + 1>(kt, kst, qf, s);
}

// O += P V for one block: 4 K-substeps of 16 keys, four 32-column fragments of d.
template <int T>
__device__ __forceinline__ void attn_pv_step(const AttnVTile& vt, const lds_char* vst, const u32x4_t (&pf)[4],
                                             f32x16_t (&o)[4]) {
  u32x4_t vb[4];
  FragLoop<0, 4, T>::run(vt, vst, vb);
#pragma unroll
  for (int f = 0; f < 4; ++f) o[f] = mfma_bf16(vb[f], pf[T], o[f]);
  if constexpr (T + 1 < 4) attn_pv_step<T + 1>(vt, vst, pf, o);
}

__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(const AttnArgs p) {
  __shared__ __attribute__((aligned(1024))) char st0[kAttnStage];
  __shared__ __attribute__((aligned(1024))) char st1[kAttnStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seq = p.seq;
  const int nqb = (seq + kAttnBQ - 1) / kAttnBQ;
  // Workgroup x is work item x / (heads * batch) of head x % heads and
  // sequence (x / heads) % batch, so the longest items of all heads go first.
  // Causal: item i is chunk c of query block qb (see attn_key_chunks);
  // otherwise block i, all keys.
  const int hb = p.heads * p.batch;
  const int item = (int)blockIdx.x / hb;
  const int head = ((int)blockIdx.x % hb) % p.heads;
  const int zb = ((int)blockIdx.x % hb) / p.heads;
  int qb = item, chunk = 0;
  if (p.causal) {
    int id = item;
    // The grid holds exactly the chunks that exist; the bound only guards the loop.
    while (chunk < p.chunks && id >= nqb - (p.kc / 2) * chunk) {
      id -= nqb - (p.kc / 2) * chunk;
      ++chunk;
    }
    if (chunk >= p.chunks) return;   // uniform across the workgroup, before any barrier
    qb = nqb - 1 - id;
  }
  const int64_t row_base = (int64_t)zb * seq;
  const int q0 = qb * kAttnBQ;
  const int wq0 = q0 + 32 * wave;                 // this wave's first query row
  const int qrow = wq0 + (lane & 31);             // this lane's query row
  const bf16_t* Kh = p.K + row_base * p.ldk + head * kAttnD;
  const bf16_t* Vh = p.V + row_base * p.ldv + head * kAttnD;

  // Q fragments: row qrow, d = 16 s + 8 h .. + 7 (zero past the sequence).
  u32x4_t qf[8];
  {
    const bf16_t* qp = p.Q + (row_base + qrow) * p.ldq + head * kAttnD + 8 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = qrow < seq ? *reinterpret_cast<const u32x4_t*>(qp + 16 * s) : u32x4_t{0u, 0u, 0u, 0u};
  }

  AttnKTile kt;
  AttnVTile vt;
  kt.init(wave, lane, p.ldk, 0);
  vt.init(wave, lane, p.ldv, 0);
  // Keys [kv0, kv0 + 64) into stage dst; rows past the sequence read as zero.
  auto issue = [&](int j, lds_char* dst) {
    const int kv0 = j * kAttnBK;
    const int rows = min(kAttnBK, seq - kv0);
    const uint32_t nk = (uint32_t)(((int64_t)(rows - 1) * p.ldk + 64) * 2);
    const uint32_t nv = (uint32_t)(((int64_t)(rows - 1) * p.ldv + kAttnD) * 2);
    kt.load(Kh + (int64_t)kv0 * p.ldk, nk, dst, wave);
    kt.load(Kh + (int64_t)kv0 * p.ldk + 64, nk, dst + AttnKTile::BYTES, wave);
    vt.load(Vh + (int64_t)kv0 * p.ldv, nv, dst + 2 * AttnKTile::BYTES, wave);
  };

  const int kv_end = p.causal ? min(seq, q0 + kAttnBQ) : seq;
  const int j0 = p.causal ? chunk * p.kc : 0;
  const int j1 = p.causal ? min((kv_end + kAttnBK - 1) / kAttnBK, j0 + p.kc) : (kv_end + kAttnBK - 1) / kAttnBK;
  float m_i = -INFINITY, l_i = 0.0f;
  f32x16_t o[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[f][v] = 0.0f;

  issue(j0, (lds_char*)st0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  // One key block in stage cur (st1 when ODD, else st0; a compile-time
  // choice, so every LDS address below is a fixed offset from a per-lane base).
  auto block = [&](const int j, auto OddC) {
    constexpr bool kOdd = decltype(OddC)::value;
    lds_char* cur = kOdd ? (lds_char*)st1 : (lds_char*)st0;
    lds_char* nxt = kOdd ? (lds_char*)st0 : (lds_char*)st1;
    if (j + 1 < j1) issue(j + 1, nxt);
    const int kv0 = j * kAttnBK;
    // A wave whose rows all precede this block (causal) has nothing to add.
    if (!(p.causal && kv0 > wq0 + 31)) {
      f32x16_t s[2];
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[f][v] = 0.0f;
      attn_qk_step<0>(kt, cur, qf, s);
      // Raw scores, masked past the sequence and above the diagonal; the
      // (positive) scale goes into the exponent's FMA, so the row maximum is
      // taken before scaling.
      const bool edge = kv0 + kAttnBK > seq || (p.causal && kv0 + kAttnBK - 1 > wq0);
      if (edge) {   // one uniform branch per block; selects inside
        const bool causal = p.causal != 0;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kv = kv0 + 32 * f + 8 * (v >> 2) + 4 * h + (v & 3);
            s[f][v] = ((kv >= seq) | (causal & (kv > qrow))) ? -INFINITY : s[f][v];
          }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, s[f][v]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32)) * p.scale_log2;   // this block's row maximum, base 2
      // The reference m_i moves only when some row of the wave exceeds it by
      // more than 8 (or has none yet): otherwise P = 2^(s - m_i) <= 256 and the
      // rescaling of l and O is skipped.  l and O are sums against the same
      // reference either way, so O = acc / l and lse = m_i + log2 l hold.
      if (__builtin_amdgcn_ballot_w64(mloc > m_i + 8.0f) != 0) {
        const float m_new = fmaxf(m_i, mloc);
        const float alpha = m_i == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_i - m_new);
        l_i *= alpha;
        m_i = m_new;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[f][v] *= alpha;
      }
      float lsum = 0.0f;
      u32x4_t pf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int f = t >> 1, g0 = 2 * (t & 1);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = 4 * g0 + e;   // groups g0 (e < 4) and g0 + 1 (e >= 4)
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[f][v], p.scale_log2, -m_i));
          lsum += pv[e];
        }
        pf[t] = swap_pack(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                          pack_bf16x2(pv[6], pv[7]));
      }
      lsum += __shfl_xor(lsum, 32);
      l_i += lsum;
      attn_pv_step<0>(vt, cur + 2 * AttnKTile::BYTES, pf, o);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // block j + 1 has landed (this wave's part)
    __syncthreads();                            // ... everyone's; and stage cur is free again
  };
  // Blocks j0, j0 + 2, ... use st0, the others st1.
  int jj = j0;
  for (; jj + 1 < j1; jj += 2) {
    block(jj, std::false_type{});
    block(jj + 1, std::true_type{});
  }
  if (jj < j1) block(jj, std::false_type{});

  // Every row of a chunk sees at least one key (chunk c starts at key
  // 64 c kc <= the block's first row), so l_i > 0 here.
  if (qrow < seq && p.causal && attn_key_chunks(qb, seq, p.kc) > 1) {
    // one of several chunks: its normalised partial and base-2 log-sum-exp in
    // this item's slot, for attn_fwd_combine_kernel
    const float inv = 1.0f / l_i;
    const int64_t slot = ((int64_t)zb * p.heads + head) * p.items + item;
    const int r = 32 * wave + (lane & 31);
    float* dst = p.o_part + slot * (kAttnBQ * kAttnD) + (int64_t)r * kAttnD + 4 * h;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4_t*>(dst + 32 * f + 8 * g) =
            f32x4_t{o[f][4 * g] * inv, o[f][4 * g + 1] * inv, o[f][4 * g + 2] * inv, o[f][4 * g + 3] * inv};
    if (h == 0) p.lse_part[slot * kAttnBQ + r] = m_i + __log2f(l_i);
  } else if (qrow < seq) {
    // O = acc / l, stored as bf16 (8 consecutive columns of d per lane and 16-byte stores)
    const float inv = 1.0f / l_i;
    bf16_t* op = p.O + (row_base + qrow) * p.ldo + head * kAttnD + 8 * h;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int g0 = 2 * pr;
        const u32x4_t w = swap_pack(pack_bf16x2(o[f][4 * g0] * inv, o[f][4 * g0 + 1] * inv),
                                    pack_bf16x2(o[f][4 * g0 + 2] * inv, o[f][4 * g0 + 3] * inv),
                                    pack_bf16x2(o[f][4 * g0 + 4] * inv, o[f][4 * g0 + 5] * inv),
                                    pack_bf16x2(o[f][4 * g0 + 6] * inv, o[f][4 * g0 + 7] * inv));
        *reinterpret_cast<u32x4_t*>(op + 32 * f + 16 * pr) = w;
      }
    if (p.lse != nullptr && h == 0)
      p.lse[(int64_t)head * p.batch * seq + row_base + qrow] = (m_i + __log2f(l_i)) * 0.69314718055994531f;
  }
}

// O and lse of the causal query blocks whose keys were split into chunks: with
// chunk c's normalised partial O_c and base-2 log-sum-exp L_c, and M = max L_c,
// O = sum_c 2^(L_c - M) O_c / sum_c 2^(L_c - M) and lse = M + log2 sum_c
// 2^(L_c - M) (in natural-log units), the chunks taken in order.  Workgroup
// (x, head, sequence) covers 16 rows of block kc / 2 + x / 8 (the first block
// with two chunks); each thread owns 8 consecutive columns of one row.
__global__ void __launch_bounds__(256) attn_fwd_combine_kernel(const AttnArgs p) {
  const int seq = p.seq;
  const int nqb = (seq + kAttnBQ - 1) / kAttnBQ;
  const int half = p.kc / 2;
  const int qb = half + (int)blockIdx.x / 8;
  const int r = 16 * ((int)blockIdx.x % 8) + (int)threadIdx.x / 16;   // row within the block
  const int c8 = 8 * ((int)threadIdx.x % 16);                          // first of 8 columns
  const int head = blockIdx.y;
  const int qrow = qb * kAttnBQ + r;
  if (qrow >= seq) return;   // no barrier below
  const int nch = attn_key_chunks(qb, seq, p.kc);
  const int64_t hslot = ((int64_t)blockIdx.z * p.heads + head) * p.items;
  // slot of chunk c of block qb: the items of chunks before c, then nqb - 1 - qb
  float mx = -INFINITY;
  int slot = nqb - 1 - qb;
  for (int c = 0; c < nch; ++c) {
    if (c > 0) slot += nqb - half * (c - 1);
    mx = fmaxf(mx, p.lse_part[(hslot + slot) * kAttnBQ + r]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sum = 0.0f;
  slot = nqb - 1 - qb;
  for (int c = 0; c < nch; ++c) {
    if (c > 0) slot += nqb - half * (c - 1);
    const float wgt = __builtin_amdgcn_exp2f(p.lse_part[(hslot + slot) * kAttnBQ + r] - mx);
    sum += wgt;
    const float* src = p.o_part + (hslot + slot) * (kAttnBQ * kAttnD) + (int64_t)r * kAttnD + c8;
    const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(src);
    const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += wgt * x0[e];
      acc[4 + e] += wgt * x1[e];
    }
  }
  const float inv = 1.0f / sum;
  const int64_t row = (int64_t)blockIdx.z * seq + qrow;
  *reinterpret_cast<u32x4_t*>(p.O + row * p.ldo + head * kAttnD + c8) =
      u32x4_t{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
              pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  if (p.lse != nullptr && c8 == 0)
    p.lse[(int64_t)head * p.batch * seq + row] = (mx + __log2f(sum)) * 0.69314718055994531f;
}

// ================================================================ backward --
// With P = softmax(S) and D_q = sum_d dO[q,d] O[q,d]: dV = P^T dO, dP = dO V^T,
// dS = P * (dP - D), dQ = dS K * scale, dK = dS^T Q * scale.  No atomics:
// after D (attn_bwd_dot_kernel), one kernel owns a block of keys and loops
// over query blocks (dK, dV), another owns a block of queries and loops over
// key blocks (dQ); both recompute P from the saved log-sum-exp.  Causal dQ
// work is cut into key chunks whose partials attn_bwd_dq_sum_kernel adds.

struct AttnBwdArgs {
  const bf16_t* Q;
  const bf16_t* K;
  const bf16_t* V;
  const bf16_t* O;
  const bf16_t* dO;
  int64_t ldq, ldk, ldv, ldo, lddo;
  const float* lse;   // [heads, T] natural log
  float* D;           // [heads, T] workspace: sum_d dO * O
  float* L2;          // [heads, T] workspace: lse * log2(e), the base-2 form the dK/dV kernel stages
  bf16_t* dQ;
  bf16_t* dK;
  bf16_t* dV;
  int64_t lddq, lddk, lddv;
  int batch, seq, heads, causal;
  float scale, scale_log2;
  float* dq_part;     // causal: [batch][heads][dq_items][128][128] fp32 partial dQ, one per work item
  int dq_chunks;      // key chunks of the longest query block (1: no partials)
  int dq_kc;          // key blocks per chunk (even)
  int dq_items;       // work items (workgroups) per (sequence, head)
};

// Causal dQ work is split along keys in the forward's chunks (attn_key_chunks).

// D[head][t] = sum over the head's 128 columns of dO * O; 16 lanes per (row, head).
// The same pass stores lse in base 2 (L2), so the dK/dV kernel, whose queries
// change every iteration, takes it ready instead of scaling it per element.
__global__ void __launch_bounds__(256) attn_bwd_dot_kernel(const AttnBwdArgs p) {
  const int64_t T = (int64_t)p.batch * p.seq;
  const int64_t item = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);   // (row, head) = (item / heads, item % heads)
  const int j = threadIdx.x & 15;
  float acc = 0.0f;
  const bool live = item < T * p.heads;
  const int64_t t = live ? item / p.heads : 0;
  const int head = live ? (int)(item % p.heads) : 0;
  if (live) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p.dO + t * p.lddo + head * kAttnD + 8 * j);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p.O + t * p.ldo + head * kAttnD + 8 * j);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc += bf16lo(a[k]) * bf16lo(b[k]) + bf16hi(a[k]) * bf16hi(b[k]);
  }
#pragma unroll
  for (int x = 8; x >= 1; x >>= 1) acc += __shfl_xor(acc, x);
  if (live && j == 0) {
    p.D[(int64_t)head * T + t] = acc;
    p.L2[(int64_t)head * T + t] = p.lse[(int64_t)head * T + t] * 1.4426950408889634f;
  }
}

// A tile of ROWS token rows x 128 of d in LDS, read two ways: 8 consecutive d
// of one row (ds_read_b128) and 4 consecutive rows of one d column through
// the transposing read (ds_read_b64_tr_b16).  Chunk q (8 values of d) of row
// r sits at position q ^ (4 (r & 3) | ((r >> 2) & 3)), which keeps both
// patterns free of bank conflicts.
template <int ROWS, int NW>
struct AttnRowTile {
  static constexpr int BYTES = ROWS * 256;
  static constexpr int SLOTS = ROWS * 16;
  static constexpr int INSTR = SLOTS / (64 * NW);
  static_assert(SLOTS % (64 * NW) == 0, "tile too small for the waves");
  uint32_t voff[INSTR];
  uint32_t kb;          // row-read base: (lane & 31) * 256
  uint32_t ksw;         // row-read swizzle of row lane & 31
  uint32_t tb[4][2];    // transposing-read bases per 32-column block F (p0, p1)

  static __device__ __forceinline__ int sw(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

  // `off`: a byte offset added to every read address (a per-wave LDS region).
  __device__ __forceinline__ void init(int wave, int lane, int64_t ld, uint32_t off = 0) {
#pragma unroll
    for (int j = 0; j < INSTR; ++j) {
      const int s = (wave * INSTR + j) * 64 + lane;
      const int r = s >> 4, q = (s & 15) ^ sw(r);
      voff[j] = (uint32_t)(((int64_t)r * ld + q * 8) * 2);
    }
    kb = (uint32_t)(lane & 31) * 256u + off;
    ksw = (uint32_t)sw(lane & 31);
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int F = 0; F < 4; ++F)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int kr = 8 * (g >> 1) + (j >> 2) + 4 * pp;     // row within a 16-row substep
        const int q = 4 * F + 2 * (g & 1) + ((j & 3) >> 1);
        tb[F][pp] = (uint32_t)(kr * 256 + ((q ^ sw(kr)) << 4) + 8 * (j & 1)) + off;
      }
  }

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

  // Row read (b fragment whose n index is the row): lane holds row 32F + (lane & 31),
  // d = 16 S + 8 (lane >> 5) .. + 7.
  template <int F, int S>
  __device__ __forceinline__ u32x4_t row(const lds_char* src, int lane) const {
    const uint32_t c = (uint32_t)(2 * S + (lane >> 5)) ^ ksw;
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(src + F * 32 * 256 + kb + (c << 4));
  }

  // Transposing read (b fragment whose k index is the row): lane holds rows
  // 16 S + 8 (lane >> 5) .. + 7 of column 32F + (lane & 31).
  template <int F, int S>
  __device__ __forceinline__ u32x4_t col(const lds_char* src) const {
    const lds_char* p0 = src + S * 16 * 256 + tb[F][0];
    const lds_char* p1 = src + S * 16 * 256 + tb[F][1];
    const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p0);
    const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p1);
    const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0);
    const u32x2_t w1 = __builtin_bit_cast(u32x2_t, v1);
    return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
  }
};

// acc[f] += B(tile rows as n) x A over the 8 d-substeps: C[m][n] with m from a, n = tile row.
// The B fragments of substep S + 2 are read while substep S multiplies, so
// the LDS latency hides behind the MFMAs.
struct NoSide {
  template <class I>
  __device__ __forceinline__ void operator()(I) const {}
};

// side(std::integral_constant<int, S>{}) runs after substep S's products are
// issued: independent VALU work placed there executes under the MFMAs.
template <int NF, int R = 3, class Tile, class Side = NoSide>
__device__ __forceinline__ void mm_rows(const Tile& t, const lds_char* src, int lane, const u32x4_t (&a)[8],
                                        f32x16_t (&acc)[NF], Side side = Side{}) {
  static_assert(R == 2 || R == 3, "ring depth in substeps");
  u32x4_t b[R][NF];
  auto fetch = [&](auto SC) {
    constexpr int S = decltype(SC)::value;
    b[S % R][0] = t.template row<0, S>(src, lane);
    if constexpr (NF >= 2) b[S % R][1] = t.template row<1, S>(src, lane);
  };
  fetch(std::integral_constant<int, 0>{});
  if constexpr (R == 3) fetch(std::integral_constant<int, 1>{});
  auto step = [&](auto SC) {
    constexpr int S = decltype(SC)::value;
    if constexpr (S + R - 1 < 8) fetch(std::integral_constant<int, S + R - 1>{});
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = mfma_bf16(b[S % R][f], a[S], acc[f]);
    side(SC);
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead: the scheduler would sink them to their use
  };
  step(std::integral_constant<int, 0>{});
  step(std::integral_constant<int, 1>{});
  step(std::integral_constant<int, 2>{});
  step(std::integral_constant<int, 3>{});
  step(std::integral_constant<int, 4>{});
  step(std::integral_constant<int, 5>{});
  step(std::integral_constant<int, 6>{});
  step(std::integral_constant<int, 7>{});
}

// acc[F] += B(tile rows as k, d block F as n) x A over NT row-substeps of 16.
// The 4 NT products run in the order (T, F); the B fragment of product i + D
// is read while product i multiplies (a ring of D + 1 fragments).
template <int NT, bool AGPR = false, int D = 4, class Tile, class Side = NoSide>
__device__ __forceinline__ void mm_cols(const Tile& t, const lds_char* src, const u32x4_t (&a)[NT],
                                        f32x16_t (&acc)[4], Side side = Side{}) {
  static_assert(NT <= 4 && D >= 1 && D <= 7, "at most 4 row-substeps");
  constexpr int N = 4 * NT, R = D + 1;
  u32x4_t b[R];
  auto fetch = [&](auto IC) {
    constexpr int I = decltype(IC)::value;
    if constexpr (I < N) b[I % R] = t.template col<I % 4, I / 4>(src);
  };
  static_for<D>(fetch);
  auto step = [&](auto IC) {
    constexpr int I = decltype(IC)::value;
    fetch(std::integral_constant<int, I + D>{});
    if constexpr (AGPR) mfma_bf16_agpr<(I % 4 == 0) ? 3 : 0>(b[I % R], a[I / 4], acc[I % 4]);  // first use of a[I/4]
    else acc[I % 4] = mfma_bf16(b[I % R], a[I / 4], acc[I % 4]);
    side(IC);
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead: the scheduler would sink them to their use
  };
  static_for<N>(step);
}

// A fragments of a 32 x 32k block held in accumulator layout (row = lane & 31,
// 4-column groups) for the k-substeps 16t .. 16t + 15, t < 2 * NF.
template <int NF>
__device__ __forceinline__ void acc_to_afrag(const float (&x)[NF][16], u32x4_t (&af)[2 * NF]) {
#pragma unroll
  for (int t = 0; t < 2 * NF; ++t) {
    const int f = t >> 1, v0 = 8 * (t & 1);
    af[t] = swap_pack(pack_bf16x2(x[f][v0], x[f][v0 + 1]), pack_bf16x2(x[f][v0 + 2], x[f][v0 + 3]),
                      pack_bf16x2(x[f][v0 + 4], x[f][v0 + 5]), pack_bf16x2(x[f][v0 + 6], x[f][v0 + 7]));
  }
}

// Stores a wave's 32 x 128 fp32 block (accumulator layout) as bf16 rows times `mul`.
__device__ __forceinline__ void store_rows_bf16(const f32x16_t (&acc)[4], float mul, bf16_t* rowp, int h) {
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int g0 = 8 * pr;
      const u32x4_t w = swap_pack(pack_bf16x2(acc[f][g0] * mul, acc[f][g0 + 1] * mul),
                                  pack_bf16x2(acc[f][g0 + 2] * mul, acc[f][g0 + 3] * mul),
                                  pack_bf16x2(acc[f][g0 + 4] * mul, acc[f][g0 + 5] * mul),
                                  pack_bf16x2(acc[f][g0 + 6] * mul, acc[f][g0 + 7] * mul));
      *reinterpret_cast<u32x4_t*>(rowp + 32 * f + 16 * pr + 8 * h) = w;
    }
}

constexpr int kAttnBwdBQ = 64;   // query rows per block in the key-stationary kernel
using AttnQTile = AttnRowTile<kAttnBwdBQ, 2>;   // 64 rows, 2 waves load it
constexpr int kAttnDkvRows = 2 * AttnQTile::BYTES;        // Q and dO tiles: 32 KB
constexpr int kAttnDkvStage = kAttnDkvRows + 2 * 256;     // + the block's 64 lse and 64 D values

// 64 consecutive floats (one per lane) from global memory into LDS through the
// buffer unit; lanes past `nbytes` read zero.
__device__ __forceinline__ void lds_dma_f32x64(const float* base, uint32_t nbytes, lds_char* dst, int lane) {
  const uint64_t addr = reinterpret_cast<uint64_t>(base);
  const i32x4_t rsrc = {(int)(uint32_t)addr, (int)((addr >> 32) & 0xffffu), (int)nbytes, kBufferWord3};
  const uint32_t voff = (uint32_t)lane * 4u;
  const uint32_t lds = (uint32_t)(uintptr_t)dst;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

constexpr int kAttnDkvStride = (kAttnDkvStage + 1023) / 1024 * 1024;   // stage pitch in LDS

// dK, dV for 64 keys of one head, over all query blocks that see them.  The
// workgroup's 4 waves form two pairs; each pair holds the 64 keys (2 waves x
// 32, K and V rows in registers as A fragments) and takes half of the query
// blocks, through its own two LDS stages; at the end the second pair's sums
// go through LDS and the first pair adds them (fixed order) and stores.  With
// one wave per SIMD (the sums and K, V need most of a SIMD's registers), a
// workgroup per key block and the halved query ranges keep every SIMD busy
// with balanced work even when causal.
__global__ void __launch_bounds__(256, 1) attn_bwd_dkdv_kernel(const AttnBwdArgs p) {
  __shared__ __attribute__((aligned(1024))) char stg[4 * kAttnDkvStride];
  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = wave >> 1, wp = wave & 1;   // pair, wave within the pair
  const int seq = p.seq;
  // Workgroup x is key block x / (heads * batch) of head x % heads and sequence
  // (x / heads) % batch: the key blocks that see the most queries (causal: the
  // first) of every head and sequence are dispatched first.
  const int hb = p.heads * p.batch;
  const int kb = (int)blockIdx.x / hb;
  const int head = ((int)blockIdx.x % hb) % p.heads;
  const int z = ((int)blockIdx.x % hb) / p.heads;
  const int64_t T = (int64_t)p.batch * seq;
  const int64_t row_base = (int64_t)z * seq;
  const int k0 = kb * 64;
  const int kw0 = k0 + 32 * wp;
  const int krow = kw0 + (lane & 31);

  u32x4_t kf[8], vf[8];
  {
    const bf16_t* kp = p.K + (row_base + krow) * p.ldk + head * kAttnD + 8 * h;
    const bf16_t* vp = p.V + (row_base + krow) * p.ldv + head * kAttnD + 8 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = krow < seq ? *reinterpret_cast<const u32x4_t*>(kp + 16 * s) : u32x4_t{0u, 0u, 0u, 0u};
      vf[s] = krow < seq ? *reinterpret_cast<const u32x4_t*>(vp + 16 * s) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  // Pair pr's stages are stg + (2 pr + parity) * stride; the pair offset goes
  // into the tiles' read bases, so reads address stg + parity * stride.
  const uint32_t pair_off = (uint32_t)(2 * pr * kAttnDkvStride);
  AttnQTile qt, ot;
  qt.init(wp, lane, p.ldq, pair_off);
  ot.init(wp, lane, p.lddo, pair_off);
  const bf16_t* Qh = p.Q + row_base * p.ldq + head * kAttnD;
  const bf16_t* dOh = p.dO + row_base * p.lddo + head * kAttnD;
  const float* lse_h = p.L2 + (int64_t)head * T + row_base;
  const float* D_h = p.D + (int64_t)head * T + row_base;
  // One stage: the query block's Q and dO tiles, then its base-2 lse and D values
  // (the pair's wave 0 fetches lse, wave 1 fetches D), all through the LDS DMA
  // so a single vmcnt wait covers the whole next stage.
  auto issue = [&](int qb, lds_char* dst) {
    const int q0 = qb * kAttnBwdBQ;
    const int rows = min(kAttnBwdBQ, seq - q0);
    qt.load(Qh + (int64_t)q0 * p.ldq, (uint32_t)(((int64_t)(rows - 1) * p.ldq + kAttnD) * 2), dst, wp);
    ot.load(dOh + (int64_t)q0 * p.lddo, (uint32_t)(((int64_t)(rows - 1) * p.lddo + kAttnD) * 2),
            dst + AttnQTile::BYTES, wp);
    lds_dma_f32x64((wp == 0 ? lse_h : D_h) + q0, (uint32_t)rows * 4u, dst + kAttnDkvRows + 256 * wp, lane);
  };

  f32x16_t dk[4], dv[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int v = 0; v < 16; ++v) dk[f][v] = dv[f][v] = 0.0f;
    // Move the sums to accumulation registers once, where the loop keeps them.
    asm volatile("" : "+a"(dk[f]));
    asm volatile("" : "+a"(dv[f]));
  }

  // Query blocks [qb0, nqb) (causal: from the key block's own), the first
  // ceil(n/2) to pair 0, the rest to pair 1; both pairs run ceil(n/2)
  // iterations (pair 1's last may be empty) so that they meet the same barriers.
  const int nqb = (seq + kAttnBwdBQ - 1) / kAttnBwdBQ;
  const int qb0 = p.causal ? k0 / kAttnBwdBQ : 0;
  const int nit = (nqb - qb0 + 1) / 2;
  const int my0 = pr == 0 ? qb0 : qb0 + nit;
  const int my1 = pr == 0 ? qb0 + nit : nqb;
  lds_char* const st = (lds_char*)stg;
  auto pstage = [&](int parity) { return st + (2 * pr + parity) * kAttnDkvStride; };   // this pair's stage
  if (my0 < my1) issue(my0, pstage(0));
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  // Iteration i: query block my0 + i in the pair's stage i & 1 (ODD; a
  // compile-time choice, so the tiles' reads are fixed offsets from their
  // per-lane bases, which carry the pair offset).
  auto block = [&](const int i, auto OddC) {
    constexpr bool kOdd = decltype(OddC)::value;
    const lds_char* cur = st + (kOdd ? kAttnDkvStride : 0);   // + pair_off inside the tiles
    lds_char* const mine = pstage(kOdd ? 1 : 0);
    const int qb = my0 + i;
    if (qb + 1 < my1) issue(qb + 1, pstage(kOdd ? 0 : 1));
    if (qb < my1) {
    const int q0 = qb * kAttnBwdBQ;
    const bool edge = q0 + kAttnBwdBQ > seq || (p.causal && q0 < kw0 + 31);
    const lds_char* lse_s = mine + kAttnDkvRows;
    const lds_char* d_s = mine + kAttnDkvRows + 256;
    // Accumulator layout: lane holds key krow and queries q0 + 32 f + 8 g + 4 h + e
    // in register 4 g + e of block f.  The VALU work runs under the MFMAs of
    // the next product: P^T under dP^T, dS^T under dV.  P^T and dS^T are kept
    // as packed bf16 pairs (pk) in accumulator layout.
    f32x16_t sacc[2], dacc[2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[f][v] = dacc[f][v] = 0.0f;
    // This block's lse and D values for the lane's queries, read before the
    // products so that no later wait on them also drains the fragment reads.
    f32x4_t l4s[8], d4s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int qo = (32 * (k / 4) + 8 * (k % 4) + 4 * h) * 4;
      l4s[k] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(lse_s + qo);
      d4s[k] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(d_s + qo);
    }
    mm_rows<2>(qt, cur, lane, kf, sacc);   // S^T = K Q^T
    if (edge) {   // masked scores -inf, so P^T = 0 there (the scale is positive); one uniform branch
      const bool causal = p.causal != 0, kout = krow >= seq;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = q0 + 32 * f + 8 * (v >> 2) + 4 * h + (v & 3);
          sacc[f][v] = ((q >= seq) | kout | (causal & (q < krow))) ? -INFINITY : sacc[f][v];
        }
    }
    uint32_t pk[2][8];
    // P^T = exp(S^T * scale - lse), slice (f, g) = (S / 4, S % 4) under substep S of dP^T
    auto p_slice = [&](auto SC) {
      constexpr int f = decltype(SC)::value / 4, g = decltype(SC)::value % 4;
      const f32x4_t l4 = l4s[4 * f + g];
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[f][4 * g + e], p.scale_log2, -l4[e]));
      pk[f][2 * g] = pack_bf16x2(pv[0], pv[1]);
      pk[f][2 * g + 1] = pack_bf16x2(pv[2], pv[3]);
    };
    mm_rows<2>(ot, cur + AttnQTile::BYTES, lane, vf, dacc, p_slice);   // dP^T = V dO^T
    u32x4_t af[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      af[t] = swap_pack(pk[t >> 1][4 * (t & 1)], pk[t >> 1][4 * (t & 1) + 1], pk[t >> 1][4 * (t & 1) + 2],
                        pk[t >> 1][4 * (t & 1) + 3]);
    // dS^T = P^T * (dP^T - D) from the bf16 P^T, slice (f, g) = (I / 8, (I / 2) % 4) under product I of dV
    auto ds_slice = [&](auto IC) {
      constexpr int I = decltype(IC)::value;
      if constexpr (I % 2 == 0) {
        constexpr int f = I / 8, g = (I / 2) % 4;
        const f32x4_t d4 = d4s[4 * f + g];
        const uint32_t p01 = pk[f][2 * g], p23 = pk[f][2 * g + 1];
        pk[f][2 * g] = pack_bf16x2(bf16lo(p01) * (dacc[f][4 * g] - d4[0]), bf16hi(p01) * (dacc[f][4 * g + 1] - d4[1]));
        pk[f][2 * g + 1] =
            pack_bf16x2(bf16lo(p23) * (dacc[f][4 * g + 2] - d4[2]), bf16hi(p23) * (dacc[f][4 * g + 3] - d4[3]));
      }
    };
    mm_cols<4, true>(ot, cur + AttnQTile::BYTES, af, dv, ds_slice);   // dV += P^T dO
#pragma unroll
    for (int t = 0; t < 4; ++t)
      af[t] = swap_pack(pk[t >> 1][4 * (t & 1)], pk[t >> 1][4 * (t & 1) + 1], pk[t >> 1][4 * (t & 1) + 2],
                        pk[t >> 1][4 * (t & 1) + 3]);
    mm_cols<4, true>(qt, cur, af, dk);   // dK += dS^T Q
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
  };
  int i = 0;
  for (; i + 1 < nit; i += 2) {
    block(i, std::false_type{});
    block(i + 1, std::true_type{});
  }
  if (i < nit) block(i, std::false_type{});
  agpr_acc_drain(dk, dv);   // the last products into dk, dv have retired before VALU reads them
  // Pair 1's sums into LDS (free: the last iteration ended with a barrier),
  // element-major so that each read and write is one dword per lane.
  float* const red = reinterpret_cast<float*>(stg);
  if (pr == 1) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        red[(wp * 128 + 16 * f + v) * 64 + lane] = dk[f][v];
        red[(wp * 128 + 64 + 16 * f + v) * 64 + lane] = dv[f][v];
      }
  }
  __syncthreads();
  if (pr == 0) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        dk[f][v] += red[(wp * 128 + 16 * f + v) * 64 + lane];
        dv[f][v] += red[(wp * 128 + 64 + 16 * f + v) * 64 + lane];
      }
    if (krow < seq) {
      store_rows_bf16(dv, 1.0f, p.dV + (row_base + krow) * p.lddv + head * kAttnD, h);
      store_rows_bf16(dk, p.scale, p.dK + (row_base + krow) * p.lddk + head * kAttnD, h);
    }
  }
}

using AttnKVTile = AttnRowTile<kAttnBK, 4>;   // 64 key rows x 128, 4 waves load it
constexpr int kAttnDqStage = 2 * AttnKVTile::BYTES;  // K and V: 32 KB

// dQ for 128 query rows of one head (4 waves x 32), over the key blocks they
// see (causal: over one key chunk, see attn_key_chunks).
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_kernel(const AttnBwdArgs p) {
  __shared__ __attribute__((aligned(1024))) char st0[kAttnDqStage];
  __shared__ __attribute__((aligned(1024))) char st1[kAttnDqStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seq = p.seq;
  const int nqb = (seq + kAttnBQ - 1) / kAttnBQ;
  // Causal: workgroup x is chunk c of query block qb, enumerated chunk by chunk
  // (c = 0 for every block, then c = 1 for the blocks that have it, ...), the
  // blocks of one chunk from the last (longest) down.  Otherwise block x, all keys.
  // The grid is item-major as in the forward: workgroup x is item
  // x / (heads * batch) of head x % heads and sequence (x / heads) % batch.
  const int hb = p.heads * p.batch;
  const int item = (int)blockIdx.x / hb;
  const int head = ((int)blockIdx.x % hb) % p.heads;
  const int zb = ((int)blockIdx.x % hb) / p.heads;
  int qb = item, chunk = 0;
  if (p.causal) {
    int id = item;
    // The grid holds exactly the chunks that exist; the bound only guards the loop.
    while (chunk < p.dq_chunks && id >= nqb - (p.dq_kc / 2) * chunk) {
      id -= nqb - (p.dq_kc / 2) * chunk;
      ++chunk;
    }
    if (chunk >= p.dq_chunks) return;   // uniform across the workgroup, before any barrier
    qb = nqb - 1 - id;
  }
  const int64_t T = (int64_t)p.batch * seq;
  const int64_t row_base = (int64_t)zb * seq;
  const int q0 = qb * kAttnBQ;
  const int wq0 = q0 + 32 * wave;
  const int qrow = wq0 + (lane & 31);

  u32x4_t qf[8], of[8];
  {
    const bf16_t* qp = p.Q + (row_base + qrow) * p.ldq + head * kAttnD + 8 * h;
    const bf16_t* op = p.dO + (row_base + qrow) * p.lddo + head * kAttnD + 8 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[s] = qrow < seq ? *reinterpret_cast<const u32x4_t*>(qp + 16 * s) : u32x4_t{0u, 0u, 0u, 0u};
      of[s] = qrow < seq ? *reinterpret_cast<const u32x4_t*>(op + 16 * s) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  const float log2e = 1.4426950408889634f;
  const float lse2 = qrow < seq ? p.lse[(int64_t)head * T + row_base + qrow] * log2e : 0.0f;
  const float Dq = qrow < seq ? p.D[(int64_t)head * T + row_base + qrow] : 0.0f;
  AttnKVTile ktile, vtile;
  ktile.init(wave, lane, p.ldk);
  vtile.init(wave, lane, p.ldv);
  const bf16_t* Kh = p.K + row_base * p.ldk + head * kAttnD;
  const bf16_t* Vh = p.V + row_base * p.ldv + head * kAttnD;
  auto issue = [&](int j, lds_char* dst) {
    const int kv0 = j * kAttnBK;
    const int rows = min(kAttnBK, seq - kv0);
    ktile.load(Kh + (int64_t)kv0 * p.ldk, (uint32_t)(((int64_t)(rows - 1) * p.ldk + kAttnD) * 2), dst, wave);
    vtile.load(Vh + (int64_t)kv0 * p.ldv, (uint32_t)(((int64_t)(rows - 1) * p.ldv + kAttnD) * 2),
               dst + AttnKVTile::BYTES, wave);
  };

  f32x16_t dq[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int v = 0; v < 16; ++v) dq[f][v] = 0.0f;
  }
  const int kv_end = p.causal ? min(seq, q0 + kAttnBQ) : seq;
  const int j0 = p.causal ? chunk * p.dq_kc : 0;
  const int j1 = p.causal ? min((kv_end + kAttnBK - 1) / kAttnBK, j0 + p.dq_kc) : (kv_end + kAttnBK - 1) / kAttnBK;
  issue(j0, (lds_char*)st0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  // One key block in stage cur (st1 when ODD, else st0; a compile-time
  // choice, so every LDS address below is a fixed offset from a per-lane base).
  auto block = [&](const int j, auto OddC) {
    constexpr bool kOdd = decltype(OddC)::value;
    lds_char* cur = kOdd ? (lds_char*)st1 : (lds_char*)st0;
    lds_char* nxt = kOdd ? (lds_char*)st0 : (lds_char*)st1;
    if (j + 1 < j1) issue(j + 1, nxt);
    const int kv0 = j * kAttnBK;
    if (!(p.causal && kv0 > wq0 + 31)) {
      const bool edge = kv0 + kAttnBK > seq || (p.causal && kv0 + kAttnBK - 1 > wq0);
      // P = exp(S * scale - lse), kept as packed bf16 pairs in accumulator
      // layout (lane: query qrow, keys kv0 + 32 f + 8 g + 4 h + e).
      uint32_t pk[2][8];
      {
        f32x16_t sacc[2];   // S = Q K^T
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int v = 0; v < 16; ++v) sacc[f][v] = 0.0f;
        mm_rows<2, 2>(ktile, cur, lane, qf, sacc);
        if (edge) {   // masked scores -inf, so P = 0 there (the scale is positive)
          const bool causal = p.causal != 0;
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int kv = kv0 + 32 * f + 8 * (v >> 2) + 4 * h + (v & 3);
              sacc[f][v] = ((kv >= seq) | (causal & (kv > qrow))) ? -INFINITY : sacc[f][v];
            }
        }
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float pv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[f][4 * g + e], p.scale_log2, -lse2));
            pk[f][2 * g] = pack_bf16x2(pv[0], pv[1]);
            pk[f][2 * g + 1] = pack_bf16x2(pv[2], pv[3]);
          }
      }
      {
        f32x16_t dacc[2];   // dP = dO V^T
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int v = 0; v < 16; ++v) dacc[f][v] = 0.0f;
        mm_rows<2, 2>(vtile, cur + AttnKVTile::BYTES, lane, of, dacc);
        // dS = P * (dP - D)
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint32_t p01 = pk[f][2 * g], p23 = pk[f][2 * g + 1];
            pk[f][2 * g] = pack_bf16x2(bf16lo(p01) * (dacc[f][4 * g] - Dq), bf16hi(p01) * (dacc[f][4 * g + 1] - Dq));
            pk[f][2 * g + 1] =
                pack_bf16x2(bf16lo(p23) * (dacc[f][4 * g + 2] - Dq), bf16hi(p23) * (dacc[f][4 * g + 3] - Dq));
          }
      }
      u32x4_t da[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        da[t] = swap_pack(pk[t >> 1][4 * (t & 1)], pk[t >> 1][4 * (t & 1) + 1], pk[t >> 1][4 * (t & 1) + 2],
                          pk[t >> 1][4 * (t & 1) + 3]);
      mm_cols<4, false, 2>(ktile, cur, da, dq);   // dQ += dS K
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
  };
  // Blocks j0, j0 + 2, ... use st0, the others st1.
  int jj = j0;
  for (; jj + 1 < j1; jj += 2) {
    block(jj, std::false_type{});
    block(jj + 1, std::true_type{});
  }
  if (jj < j1) block(jj, std::false_type{});
  if (p.causal && attn_key_chunks(qb, seq, p.dq_kc) > 1) {
    // one of several chunks: its fp32 partial (unscaled) in this item's slot, for attn_bwd_dq_sum_kernel
    float* dst = p.dq_part +
                 (((int64_t)zb * p.heads + head) * p.dq_items + item) * (kAttnBQ * kAttnD) +
                 (int64_t)(32 * wave + (lane & 31)) * kAttnD + 4 * h;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4_t*>(dst + 32 * f + 8 * g) =
            f32x4_t{dq[f][4 * g], dq[f][4 * g + 1], dq[f][4 * g + 2], dq[f][4 * g + 3]};
  } else if (qrow < seq) {
    store_rows_bf16(dq, p.scale, p.dQ + (row_base + qrow) * p.lddq + head * kAttnD, h);
  }
}

// dQ of the causal query blocks that were split into several key chunks: the
// chunks' partials added in chunk order, scaled, rounded to bf16.  Workgroup
// (x, head, sequence) covers 16 rows of block kc / 2 + x / 8 (the first block
// with two chunks); each thread owns 8 consecutive columns of one row.
__global__ void __launch_bounds__(256) attn_bwd_dq_sum_kernel(const AttnBwdArgs p) {
  const int seq = p.seq;
  const int nqb = (seq + kAttnBQ - 1) / kAttnBQ;
  const int half = p.dq_kc / 2;
  const int qb = half + (int)blockIdx.x / 8;
  const int r = 16 * ((int)blockIdx.x % 8) + (int)threadIdx.x / 16;   // row within the block
  const int c8 = 8 * ((int)threadIdx.x % 16);                          // first of 8 columns
  const int head = blockIdx.y;
  const int nch = attn_key_chunks(qb, seq, p.dq_kc);
  const float* base = p.dq_part + ((int64_t)blockIdx.z * p.heads + head) * p.dq_items * (kAttnBQ * kAttnD) +
                      r * kAttnD + c8;
  // slot of chunk c of block qb: the items of chunks before c, then nqb - 1 - qb
  int slot = nqb - 1 - qb;
  const float* src = base + (int64_t)slot * (kAttnBQ * kAttnD);
  f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(src);
  f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(src + 4);
  for (int c = 1; c < nch; ++c) {
    slot += nqb - half * (c - 1);
    const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(base + (int64_t)slot * (kAttnBQ * kAttnD));
    const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(base + (int64_t)slot * (kAttnBQ * kAttnD) + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a0[e] += x0[e];
      a1[e] += x1[e];
    }
  }
  const int q = qb * kAttnBQ + r;
  if (q < seq) {
    const float sc = p.scale;
    *reinterpret_cast<u32x4_t*>(p.dQ + ((int64_t)blockIdx.z * seq + q) * p.lddq + head * kAttnD + c8) =
        u32x4_t{pack_bf16x2(a0[0] * sc, a0[1] * sc), pack_bf16x2(a0[2] * sc, a0[3] * sc),
                pack_bf16x2(a1[0] * sc, a1[1] * sc), pack_bf16x2(a1[2] * sc, a1[3] * sc)};
  }
}

}  // namespace tpmlp
