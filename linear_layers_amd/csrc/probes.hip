// Machine probes behind the GEMM design's bounds: how many bytes per clock one
// CU's load path moves into LDS for the operand patterns of a 256x256 tile,
// and how fast LDS returns fragment reads at a given number of waves.  They
// measure the hardware, not the library: nothing here computes a product, and
// libtpmlp.so does not contain this file.  Built as libtpmlp_probe.so;
// include/tpmlp_probe.h declares the calls.
//
// Load-path probe.  256 workgroups of 4 waves, one per CU, each moving the
// operand tiles of one 256x256 output tile for 64 K steps of 64 (64 KB per CU
// per step: A is 256 K-contiguous rows x 128 B, B is 64 N-contiguous K-rows x
// 512 B).  Workgroup g takes row block g % 32 of A (8192 x lda bf16) and
// column block g / 32 of B (4096 x ldb bf16, after A).  A step's 16 loads per
// wave, by pattern:
//   0  the kernel's mix: 8 loads of A (8 rows x 128 B each), 8 of B (2 K-rows x 512 B)
//   1  A only (two K steps' worth of A)
//   2  B only
//   3  A only, the 8 rows of one load 32 rows apart
// and by mode:
//   0  buffer_load_dwordx4 ... lds (LDS DMA), the next step's loads issued
//      before waiting for this step's
//   1  global_load_dwordx4 into registers, two steps in flight, consumed by XOR
//   2  as 1, then written to a two-stage LDS ring with ds_write_b128 and a
//      barrier per step
// Every address the kernels form is checked on the host against the buffer
// before the launch.
//
// LDS-read probe.  256 workgroups (one per CU, 96 KB of LDS each) of W waves,
// each issuing groups of 8 independent reads (ds_read_b128: 1 KB a read, or
// ds_read_b64_tr_b16: 512 B) at conflict-free addresses, then waiting for the
// group; B/clk per CU from the shader-clock counter of workgroup 0.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/tpmlp_probe.h"

namespace {

typedef int i32x4_p __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_p __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_p __attribute__((ext_vector_type(2)));

constexpr int kWg = 256, kSteps = 64, kRowsA = 8192, kRowsB = 4096;
constexpr double kStepBytes = 65536.0;   // per CU per step

char g_err[256];

int fail(const char* what, hipError_t e) {
  snprintf(g_err, sizeof g_err, "%s: %s", what, hipGetErrorString(e));
  return 1;
}

__host__ __device__ inline bool load_is_b(int pat, int j) { return pat == 0 ? j >= 8 : pat == 2; }
// K step (0..63) of load j at step st.
__host__ __device__ inline int load_kstep(int pat, int j, int st) { return pat == 0 ? st : (2 * st + (j >> 3)) & 63; }

// Byte offset of lane's 16 bytes of load j, step st.
__host__ __device__ inline uint64_t probe_offset(int pat, int wg, int wave, int j, int lane, int st, int lda, int ldb) {
  const int slot = (wave * 8 + (j & 7)) * 64 + lane;   // 0 .. 2047: 16-byte chunks of one operand's step
  const int ks = load_kstep(pat, j, st);
  if (!load_is_b(pat, j)) {
    int row = slot / 8;
    if (pat == 3) row = (row % 8) * 32 + row / 8;
    row += (wg % 32) * 256;
    return ((uint64_t)row * lda + ks * 64 + (slot % 8) * 8) * 2;
  }
  const int k = slot / 32, q = slot % 32;
  return (uint64_t)kRowsA * lda * 2 + ((uint64_t)(ks * 64 + k) * ldb + (wg / 32) * 256 + q * 8) * 2;
}

// Bytes between load j's addresses at consecutive K steps.
__host__ __device__ inline uint32_t kstep_bytes(int pat, int j, int ldb) {
  return load_is_b(pat, j) ? 64u * ldb * 2 : 128u;
}

template <int MODE, int PAT>
__global__ void __launch_bounds__(256, 1) load_probe(const char* g, uint64_t bytes, int lda, int ldb, int* sink,
                                                     unsigned long long* clk) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * 65536];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x;
  unsigned long long c0 = 0, r0 = 0;
  if (wg == 0 && tid == 0) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  int acc = 0;
  if constexpr (MODE == 0) {
    const uint64_t base = reinterpret_cast<uint64_t>(g);
    const i32x4_p rsrc = {(int)(uint32_t)base, (int)((base >> 32) & 0xffff), (int)(uint32_t)bytes, 0x00020000};
    uint32_t v0[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v0[j] = (uint32_t)probe_offset(PAT, wg, wave, j, lane, 0, lda, ldb);
    for (int st = 0; st < kSteps; ++st) {
      char* dst = lds + (st & 1) * 65536;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t m0 = (uint32_t)(uintptr_t)(dst + (wave * 16 + j) * 1024);
        const uint32_t off = v0[j] + (uint32_t)(load_kstep(PAT, j, st) - load_kstep(PAT, j, 0)) * kstep_bytes(PAT, j, ldb);
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(m0), "v"(off), "s"(rsrc)
                     : "memory", "m0");
      }
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      __syncthreads();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    acc = lds[tid];
  } else {
    i32x4_p b0[16], b1[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      b0[j] = *reinterpret_cast<const i32x4_p*>(g + probe_offset(PAT, wg, wave, j, lane, 0, lda, ldb));
    i32x4_p x = {0, 0, 0, 0};
    for (int st = 0; st < kSteps; st += 2) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        b1[j] = *reinterpret_cast<const i32x4_p*>(g + probe_offset(PAT, wg, wave, j, lane, st + 1, lda, ldb));
      if constexpr (MODE == 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) x ^= b0[j];
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) *reinterpret_cast<i32x4_p*>(lds + (wave * 16 + j) * 1024 + lane * 16) = b0[j];
        __syncthreads();
      }
      if (st + 2 < kSteps) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          b0[j] = *reinterpret_cast<const i32x4_p*>(g + probe_offset(PAT, wg, wave, j, lane, st + 2, lda, ldb));
      }
      if constexpr (MODE == 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) x ^= b1[j];
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          *reinterpret_cast<i32x4_p*>(lds + 65536 + (wave * 16 + j) * 1024 + lane * 16) = b1[j];
        __syncthreads();
      }
    }
    if constexpr (MODE == 1) {   // touch LDS so that the occupancy matches the other modes
      lds[tid] = (char)x[0];
      lds[65536 + tid] = (char)x[1];
      __syncthreads();
    }
    acc = lds[tid] + lds[65536 + tid];
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  sink[wg * 256 + tid] = acc;
  if (wg == 0 && tid == 0) {
    clk[0] = __builtin_amdgcn_s_memtime() - c0;
    clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

template <bool B128, int NW>
__global__ void __launch_bounds__(NW * 64, 1) lds_probe(unsigned* sink, unsigned long long* clk, int iters) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[96 * 1024];
  for (int i = threadIdx.x; i < 96 * 1024 / 4; i += NW * 64) reinterpret_cast<unsigned*>(lds)[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // wave w reads the 8 KB window (w mod 8): 8 reads 1 KB (b128) or 512 B (tr) apart
  const unsigned base = (unsigned)(uintptr_t)lds + (unsigned)(wave % 8) * 8192u + (B128 ? lane * 16u : lane * 8u);
  unsigned long long c0 = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) c0 = __builtin_amdgcn_s_memtime();
  u32x4_p acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    if constexpr (B128) {
      u32x4_p v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile(
          "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\tds_read_b128 %2, %8 offset:2048\n\t"
          "ds_read_b128 %3, %8 offset:3072\n\tds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
          "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\ts_waitcnt lgkmcnt(0)"
          : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
          : "v"(base)
          : "memory");
      acc ^= v0 ^ v1 ^ v2 ^ v3 ^ v4 ^ v5 ^ v6 ^ v7;
    } else {
      u32x2_p v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %8 offset:512\n\tds_read_b64_tr_b16 %2, %8 offset:1024\n\t"
          "ds_read_b64_tr_b16 %3, %8 offset:1536\n\tds_read_b64_tr_b16 %4, %8 offset:2048\n\t"
          "ds_read_b64_tr_b16 %5, %8 offset:2560\n\tds_read_b64_tr_b16 %6, %8 offset:3072\n\t"
          "ds_read_b64_tr_b16 %7, %8 offset:3584\n\ts_waitcnt lgkmcnt(0)"
          : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
          : "v"(base)
          : "memory");
      const u32x2_p x = v0 ^ v1 ^ v2 ^ v3 ^ v4 ^ v5 ^ v6 ^ v7;
      acc[0] ^= x[0];
      acc[1] ^= x[1];
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) clk[0] = __builtin_amdgcn_s_memtime() - c0;
  sink[blockIdx.x * NW * 64 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

typedef void (*LoadKernel)(const char*, uint64_t, int, int, int*, unsigned long long*);

LoadKernel load_kernel(int mode, int pat) {
#define PROBE_CASE(M, P) \
  if (mode == M && pat == P) return load_probe<M, P>;
  PROBE_CASE(0, 0) PROBE_CASE(0, 1) PROBE_CASE(0, 2) PROBE_CASE(0, 3)
  PROBE_CASE(1, 0) PROBE_CASE(1, 1) PROBE_CASE(1, 2) PROBE_CASE(1, 3)
  PROBE_CASE(2, 0) PROBE_CASE(2, 1) PROBE_CASE(2, 2) PROBE_CASE(2, 3)
#undef PROBE_CASE
  return nullptr;
}

}  // namespace

extern "C" {

const char* tpmlp_probe_last_error(void) { return g_err; }

int tpmlp_probe_load_path(int mode, int pattern, int lda, int ldb, int reps, double* out) {
  g_err[0] = 0;
  const LoadKernel kern = load_kernel(mode, pattern);
  if (kern == nullptr || out == nullptr || reps < 1 || lda < 4096 || ldb < 2048 || lda > 65536 || ldb > 65536) {
    snprintf(g_err, sizeof g_err, "bad arguments (mode 0-2, pattern 0-3, lda >= 4096, ldb >= 2048, reps >= 1)");
    return 2;
  }
  const uint64_t bytes = (uint64_t)kRowsA * lda * 2 + (uint64_t)kRowsB * ldb * 2;
  // every address the launch forms, against the buffer (and the 32-bit offset of the DMA loads)
  uint64_t mx = 0;
  for (int wg = 0; wg < kWg; ++wg)
    for (int w = 0; w < 4; ++w)
      for (int j = 0; j < 16; ++j)
        for (int st = 0; st < kSteps; ++st)
          for (int l = 0; l < 64; ++l) {
            const uint64_t a = probe_offset(pattern, wg, w, j, l, st, lda, ldb);
            if (a > mx) mx = a;
          }
  if (mx + 16 > bytes || mx + 16 > 0xffffffffull) {
    snprintf(g_err, sizeof g_err, "probe address %llu outside the %llu-byte buffer", (unsigned long long)mx,
             (unsigned long long)bytes);
    return 3;
  }
  char* g = nullptr;
  int* sink = nullptr;
  unsigned long long* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  hipError_t e = hipMalloc(&g, bytes);
  if (e == hipSuccess) e = hipMemset(g, 1, bytes);
  if (e == hipSuccess) e = hipMalloc(&sink, kWg * 256 * sizeof(int));
  if (e == hipSuccess) e = hipMalloc(&clk, 2 * sizeof(unsigned long long));
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    for (int i = 0; i < 3; ++i) hipLaunchKernelGGL(kern, dim3(kWg), dim3(256), 0, 0, g, bytes, lda, ldb, sink, clk);
    e = hipEventRecord(e0, 0);
    for (int i = 0; i < reps && e == hipSuccess; ++i)
      hipLaunchKernelGGL(kern, dim3(kWg), dim3(256), 0, 0, g, bytes, lda, ldb, sink, clk);
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipGetLastError();
  }
  float ms = 0.f;
  unsigned long long c[2] = {0, 0};
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e == hipSuccess) e = hipMemcpy(c, clk, sizeof c, hipMemcpyDeviceToHost);
  if (e != hipSuccess) {
    rc = fail("load probe", e);
  } else {
    const double us = ms * 1e3 / reps;
    const double ghz = c[1] ? (double)c[0] / ((double)c[1] * 10.0) : 0.0;   // memrealtime ticks at 100 MHz
    const double per_cu = kSteps * kStepBytes;
    out[0] = us;
    out[1] = ghz;
    out[2] = kWg * per_cu / (us * 1e3);   // GB/s
    out[3] = ghz > 0 ? per_cu / (us * 1e3 * ghz) : 0.0;   // B/clk per CU
  }
  if (e1) (void)hipEventDestroy(e1);
  if (e0) (void)hipEventDestroy(e0);
  (void)hipFree(clk);
  (void)hipFree(sink);
  (void)hipFree(g);
  return rc;
}

int tpmlp_probe_lds_read(int transposing, int waves, int iters, double* out) {
  g_err[0] = 0;
  if ((waves != 4 && waves != 8 && waves != 16) || iters < 1 || out == nullptr) {
    snprintf(g_err, sizeof g_err, "bad arguments (waves 4, 8 or 16; iters >= 1)");
    return 2;
  }
  // addresses: window (w mod 8) * 8 KB + lane * 16 (or 8) + up to 7 KB (3.5 KB) < 64 KB of the 96 KB
  static_assert(7 * 8192 + 63 * 16 + 7168 + 16 <= 96 * 1024, "LDS probe window");
  unsigned* sink = nullptr;
  unsigned long long* clk = nullptr;
  int rc = 0;
  hipError_t e = hipMalloc(&sink, kWg * 16 * 64 * sizeof(unsigned));
  if (e == hipSuccess) e = hipMalloc(&clk, sizeof(unsigned long long));
  if (e == hipSuccess) {
    for (int i = 0; i < 2; ++i) {
      if (transposing) {
        if (waves == 4) hipLaunchKernelGGL((lds_probe<false, 4>), dim3(kWg), dim3(256), 0, 0, sink, clk, iters);
        if (waves == 8) hipLaunchKernelGGL((lds_probe<false, 8>), dim3(kWg), dim3(512), 0, 0, sink, clk, iters);
        if (waves == 16) hipLaunchKernelGGL((lds_probe<false, 16>), dim3(kWg), dim3(1024), 0, 0, sink, clk, iters);
      } else {
        if (waves == 4) hipLaunchKernelGGL((lds_probe<true, 4>), dim3(kWg), dim3(256), 0, 0, sink, clk, iters);
        if (waves == 8) hipLaunchKernelGGL((lds_probe<true, 8>), dim3(kWg), dim3(512), 0, 0, sink, clk, iters);
        if (waves == 16) hipLaunchKernelGGL((lds_probe<true, 16>), dim3(kWg), dim3(1024), 0, 0, sink, clk, iters);
      }
    }
    e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipGetLastError();
  }
  unsigned long long c = 0;
  if (e == hipSuccess) e = hipMemcpy(&c, clk, sizeof c, hipMemcpyDeviceToHost);
  if (e != hipSuccess) {
    rc = fail("LDS probe", e);
  } else {
    const double bytes = (double)iters * 8 * (transposing ? 512.0 : 1024.0) * waves;   // per CU
    out[0] = (double)c;
    out[1] = c ? bytes / (double)c : 0.0;
  }
  (void)hipFree(clk);
  (void)hipFree(sink);
  return rc;
}

}  // extern "C"
