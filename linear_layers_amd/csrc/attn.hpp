// Attention core of one shard's heads on gfx950: O = softmax(Q K^T * scale) V
// per head and sequence (optional causal mask), computed flash-style: a
// workgroup owns 128 query rows of one head, streams the keys and values in
// blocks of 64 through LDS and keeps a running row maximum and sum (the
// online softmax of sunjinbo.space/document/parallelism.html, CP · 上下文并行:
// a query block's attention accumulated key block by key block).  Heads are
// independent (damodev.csdn.net/6a43867610ee7a33f284fb9e.html, 1.2.2; the
// head-sharded projections on io.zouht.com/197.html, 2.2.1), so the grid is
// (query blocks, heads, batch).
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
};

constexpr int kAttnD = 128;   // head_dim
constexpr int kAttnBQ = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kAttnBK = 64;   // keys per block
using AttnKTile = Bf16Tile<kAttnBK, true, 64, 4>;   // 64 keys x 64 of d, K-contiguous
using AttnVTile = Bf16Tile<kAttnD, false, 64, 4>;   // 64 key rows x 128 of d, d contiguous
constexpr int kAttnStage = 2 * AttnKTile::BYTES + AttnVTile::BYTES;  // 32 KB

__device__ __forceinline__ f32x16_t mfma_bf16(const u32x4_t& b, const u32x4_t& a, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b), __builtin_bit_cast(bf16x8_t, a),
                                                  c, 0, 0, 0);
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
  const int qb = p.causal ? nqb - 1 - (int)blockIdx.x : (int)blockIdx.x;  // longest rows first when causal
  const int head = blockIdx.y;
  const int64_t row_base = (int64_t)blockIdx.z * seq;
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
  const int nkb = (kv_end + kAttnBK - 1) / kAttnBK;
  float m_i = -INFINITY, l_i = 0.0f;
  f32x16_t o[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[f][v] = 0.0f;

  issue(0, (lds_char*)st0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  for (int j = 0; j < nkb; ++j) {
    lds_char* cur = (j & 1) ? (lds_char*)st1 : (lds_char*)st0;
    lds_char* nxt = (j & 1) ? (lds_char*)st0 : (lds_char*)st1;
    if (j + 1 < nkb) issue(j + 1, nxt);
    const int kv0 = j * kAttnBK;
    // A wave whose rows all precede this block (causal) has nothing to add.
    if (!(p.causal && kv0 > wq0 + 31)) {
      f32x16_t s[2];
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[f][v] = 0.0f;
      attn_qk_step<0>(kt, cur, qf, s);
      // scores in base-2 units, masked past the sequence and above the diagonal
      const bool edge = kv0 + kAttnBK > seq || (p.causal && kv0 + kAttnBK - 1 > wq0);
      float mloc = -INFINITY;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = s[f][v] * p.scale_log2;
          if (edge) {
            const int kv = kv0 + 32 * f + 8 * (v >> 2) + 4 * h + (v & 3);
            if (kv >= seq || (p.causal && kv > qrow)) x = -INFINITY;
          }
          s[f][v] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_i, mloc);
      const float alpha = m_i == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_i - m_new);
      float lsum = 0.0f;
      u32x4_t pf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int f = t >> 1, g0 = 2 * (t & 1);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = 4 * g0 + e;   // groups g0 (e < 4) and g0 + 1 (e >= 4)
          pv[e] = __builtin_amdgcn_exp2f(s[f][v] - m_new);
          lsum += pv[e];
        }
        pf[t] = swap_pack(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                          pack_bf16x2(pv[6], pv[7]));
      }
      lsum += __shfl_xor(lsum, 32);
      l_i = l_i * alpha + lsum;
      m_i = m_new;
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[f][v] *= alpha;
      attn_pv_step<0>(vt, cur + 2 * AttnKTile::BYTES, pf, o);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // block j + 1 has landed (this wave's part)
    __syncthreads();                            // ... everyone's; and stage cur is free again
  }

  // O = acc / l, stored as bf16 (8 consecutive columns of d per lane and 16-byte stores)
  if (qrow < seq) {
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

}  // namespace tpmlp
