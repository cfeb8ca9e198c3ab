/*
 * tpmlp.h - C ABI of libtpmlp: one GPU's share of the tensor-parallel MLP
 * block (and of the head-sharded attention projections) on AMD MI355X
 * (gfx950).
 *
 * Pages cited (address, title, section):
 *   [csdn]   damodev.csdn.net/6a43867610ee7a33f284fb9e.html, 1 张量并行
 *            (1.1 矩阵分块乘法: 列切分 / 外积和切分; 1.2.1 MLP 模块的张量并行)
 *   [zouht]  io.zouht.com/197.html, 2 张量并行 (2.1 概念, the two block
 *            equations; 2.2.1 在 LLM 中的应用方式; 2.3 代价, f and f*)
 *   [wangyu] wangyu.me/posts/llm/tensor-parallelism/, 大语言模型并行策略（三）：
 *            张量并行 (两种切分方式: 按列切分, 按行切分; 通信模式;
 *            注意力机制中的张量并行; 多层感知机（MLP）中的张量并行)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - A linear layer is Y = X W with X of shape T x K (T tokens) and W of shape
 *   K x N [wangyu 两种切分方式].  A column shard of W is K x N/tp (contiguous
 *   columns i*N/tp .. (i+1)*N/tp-1); a row shard is K/tp x N (contiguous rows)
 *   [wangyu 按列切分, 按行切分; zouht 2.1].
 * - Every matrix is row-major.  A matrix argument M comes with a leading
 *   dimension ldm (elements between consecutive rows), so a shard may be a
 *   view into the full matrix (ldw = N for a column shard of W) or a packed
 *   copy (ldw = N/tp).  The buffer must hold rows x ldm elements.
 * - dtype is the storage type of inputs, weights and typed outputs:
 *   TPMLP_BF16 (bfloat16 bits, uint16) or TPMLP_F32.  Products accumulate in
 *   fp32.  Partial sums and all gradients of weights and inputs that get
 *   summed are fp32.  Conversion to bf16 rounds to nearest even.
 * - All matrix pointers are DEVICE pointers owned by the caller; the library
 *   never allocates, frees or retains them.  The library's own device memory
 *   is the workspace the caller passes, except for two allocations it makes
 *   and keeps until the process ends: the first tpmlp_profile_enable
 *   hipMallocs a small clock buffer (the profiler only), and
 *   tp_mlp_bwd_noalloc's scratch is a static device array (no allocation).  stream is a hipStream_t passed
 *   as void* (NULL = the null stream).  Work is enqueued asynchronously on
 *   it; the library never synchronises the stream.  Calls on one stream run
 *   in order; calls on different streams that share an output race.
 * - Every call validates its arguments on the host before it enqueues
 *   anything.  On any error nothing is launched and no output is touched.
 *   A kernel that fails at run time surfaces at the caller's next
 *   synchronisation; a failed launch returns TPMLP_E_HIP.
 * - Validation rules (status returned):
 *     NULL required pointer                                -> TPMLP_E_NULL
 *     tp_size < 1, or a split width not divisible by tp_size
 *       (the pages' rule that heads or columns must divide evenly
 *       [zouht 2.2.1])                                     -> TPMLP_E_DIVISIBILITY
 *     T < 0, any other size < 1, ld < row width            -> TPMLP_E_SHAPE
 *     a row width or ld not a multiple of 8 (bf16) or 4
 *       (fp32), or a pointer not 16-byte aligned           -> TPMLP_E_ALIGNMENT
 *     unknown dtype / activation                           -> TPMLP_E_DTYPE / TPMLP_E_ACT
 *     workspace too small                                  -> TPMLP_E_WORKSPACE
 *     sizes beyond 2^31-1 elements per dimension, or any
 *       leading dimension of 2^22 elements or more (a GEMM
 *       tile's byte offsets are 32-bit)                    -> TPMLP_E_SHAPE
 *   T == 0 (an empty batch) is valid: forward calls enqueue nothing; backward
 *   calls write zeros to the weight and bias gradients (sums over no rows).
 * - Status detail: tpmlp_last_error() returns a thread-local message about
 *   the last non-OK status of the calling thread.
 */
#ifndef TPMLP_H
#define TPMLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TPMLP_OK = 0,
  TPMLP_E_NULL = 1,
  TPMLP_E_SHAPE = 2,
  TPMLP_E_DIVISIBILITY = 3,
  TPMLP_E_ALIGNMENT = 4,
  TPMLP_E_DTYPE = 5,
  TPMLP_E_ACT = 6,
  TPMLP_E_WORKSPACE = 7,
  TPMLP_E_HIP = 8,
  TPMLP_E_VALUE = 9   /* a scalar argument outside its range (dropout probability, eps) */
} tpmlp_status;

typedef enum { TPMLP_F32 = 0, TPMLP_BF16 = 1 } tpmlp_dtype;

/* The elementwise activation between the two layers: the pages name ReLU or
 * GeLU [csdn 1.2.1]; GeLU is used in its tanh form,
 * gelu(x) = x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
typedef enum { TPMLP_ACT_NONE = 0, TPMLP_ACT_GELU_TANH = 1 } tpmlp_act;

/* Column-parallel layer, shard i:  H_i = X W_i + b_i,  Y_i = Act(H_i).
 * [zouht 2.1 first equation; wangyu 按列切分; csdn 1.1 列切分]
 *   X          [T, K], ldx >= K           full input (every shard sees all of X)
 *   W_shard    [K, N/tp], ldw >= N/tp     column shard i of W [K, N]
 *   bias_shard [N/tp] or NULL             slice i of the bias, added before Act
 *   Y_shard    [T, N/tp], ldy >= N/tp     output, storage dtype
 *   H_save     [T, N/tp] or NULL, ldh     pre-activation H_i, storage dtype
 *                                         (kept for the backward pass)
 * N is the full (unsharded) width; N % tp_size must be 0. */
int column_parallel_fwd(void* stream, int dtype, int act, int64_t T, int64_t K, int64_t N,
                        int tp_size, const void* X, int64_t ldx, const void* W_shard, int64_t ldw,
                        const void* bias_shard, void* Y_shard, int64_t ldy, void* H_save,
                        int64_t ldh);

/* Row-parallel layer, shard i:  Z_i = X_i W_i, an fp32 partial of full size.
 * [zouht 2.1 second equation; wangyu 按行切分; csdn 1.1 外积和切分]
 *   X_shard    [T, K/tp], ldx >= K/tp     column block i of the layer input
 *   W_shard    [K/tp, N], ldw >= N        row shard i of W [K, N]
 *   Z_partial  [T, N] fp32, ldz >= N      this shard's partial; the layer
 *                                         output is the sum over shards
 * K is the full reduction width; K % tp_size must be 0. */
int row_parallel_fwd(void* stream, int dtype, int64_t T, int64_t K, int64_t N, int tp_size,
                     const void* X_shard, int64_t ldx, const void* W_shard, int64_t ldw,
                     float* Z_partial, int64_t ldz);

/* out = sum over i < tp_size of partials[i], added in ascending i in fp32.
 * This is the local arithmetic of the All-Reduce that ends a row-parallel
 * layer (f* in the forward pass, f in the backward) [zouht 2.3; wangyu
 * 通信模式]; here all partials sit in this GPU's memory, no collective runs.
 *   partials   element (i, r, c) at partials[i*shard_stride + r*ldp + c]
 *   out        [T, N] fp32, ldo >= N; may alias partial 0 exactly
 *              (partials == out and ldp == ldo), not any other partial.
 * T rows may be a sub-range of a larger partial (pass offset pointers), which
 * is one GPU's share of a reduce-scatter. */
int shard_partial_sum(void* stream, int tp_size, int64_t T, int64_t N, const float* partials,
                      int64_t shard_stride, int64_t ldp, float* out, int64_t ldo);

/* One shard of the MLP block Z = GeLU(X W1 + b1) W2, with W1 split by
 * columns and W2 by rows so the activation output is already the row-split
 * input of the second layer [csdn 1.2.1; zouht 2.2.1 前馈网络; wangyu 多层感知机
 * （MLP）中的张量并行].  Fs = F / tp_size.
 *   X          [T, h] (ld h)
 *   W1_shard   [h, Fs], ldw1 >= Fs (ldw1 = F for a view into W1)
 *   b1_shard   [Fs] or NULL
 *   W2_shard   [Fs, h] (ld h): rows i*Fs.. of W2 [F, h]
 *   H_save     [T, Fs] or NULL (ld Fs): pre-activation, storage dtype
 *   A_save     [T, Fs] (ld Fs): activation output, storage dtype
 *   Z_partial  [T, h] fp32 (ld h): this shard's partial of Z */
int tp_mlp_fwd(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size,
               const void* X, const void* W1_shard, int64_t ldw1, const void* b1_shard,
               const void* W2_shard, void* H_save, void* A_save, float* Z_partial);

/* Bytes of device workspace tp_mlp_bwd needs for these sizes (0 on bad args). */
size_t tpmlp_bwd_workspace_bytes(int dtype, int64_t T, int64_t h, int64_t F, int tp_size);

/* One shard's backward of the MLP block for the upstream gradient dZ of the
 * block output.  Every row shard receives the same dZ because Z is the sum of
 * the partials [wangyu 按行切分, backward]; the input gradient of the
 * column-split layer is a sum over shards [wangyu 按列切分, backward; zouht
 * 2.3, f in the backward pass].  With dA_i = dZ W2_i^T and
 * dH_i = dA_i * GeLU'(H_i):
 *   dX_partial [T, h] fp32     dH_i W1_i^T (sum over shards = dX)
 *   dW1_shard  [h, Fs] fp32    X^T dH_i   (W1's orientation, ld Fs)
 *   db1_shard  [Fs] fp32 / NULL column sums of dH_i (before bf16 rounding)
 *   dW2_shard  [Fs, h] fp32    A_i^T dZ   (W2's orientation, ld h)
 * Inputs: X, W1_shard (ldw1), W2_shard, H_save and A_save from tp_mlp_fwd, and
 * dZ [T, h] in the storage dtype.  workspace: device memory of at least
 * tpmlp_bwd_workspace_bytes() bytes, 256-byte aligned, owned by the caller. */
int tp_mlp_bwd(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size,
               const void* X, const void* W1_shard, int64_t ldw1, const void* W2_shard,
               const void* H_save, const void* A_save, const void* dZ, float* dX_partial,
               float* dW1_shard, float* db1_shard, float* dW2_shard, void* workspace,
               size_t workspace_bytes);

/* The epilogues of the column-parallel layer as standalone elementwise
 * passes over an fp32 product, for the fusion ablation (the GEMM entry points
 * fuse both into the product's epilogue).  GeLU is elementwise, so it
 * commutes with the column split [csdn 1.2.1 MLP 模块的张量并行; zouht 2.2.1]
 * and each shard applies it to its own columns; the tanh form as in
 * column_parallel_fwd.
 *   bias_gelu_fwd:  A_out = GeLU(Hin + bias), H_out = Hin + bias (if not NULL)
 *     Hin [T, N] fp32 (ldin); bias [N] storage dtype or NULL; A_out, H_out
 *     [T, N] storage dtype (lda, ldh).
 *   gelu_bwd:       dH_out = dA * GeLU'(H)
 *     dA [T, N] fp32 (ldda); H [T, N] storage dtype (ldh) as saved by the
 *     forward; dH_out [T, N] storage dtype (lddh).
 * N must be a multiple of 8 (TPMLP_E_ALIGNMENT otherwise); the other rules
 * are the shared conventions above.  HBM-bound: 4 + 2 x element-size bytes
 * per element. */
int bias_gelu_fwd(void* stream, int dtype, int64_t T, int64_t N, const float* Hin, int64_t ldin,
                  const void* bias, void* A_out, int64_t lda, void* H_out, int64_t ldh);
int gelu_bwd(void* stream, int dtype, int64_t T, int64_t N, const float* dA, int64_t ldda, const void* H,
             int64_t ldh, void* dH_out, int64_t lddh);

/* tp_mlp_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same operands, outputs and results as tp_mlp_bwd
 * (the same kernels in the same order); the workspace is a static device
 * array of tpmlp_noalloc_scratch_bytes() bytes (64 MiB) that the library
 * holds on each device it runs on until the process ends.  The call makes no
 * allocation.  Sizes whose workspace (tpmlp_bwd_workspace_bytes) exceeds the
 * array return TPMLP_E_WORKSPACE before anything is enqueued (a 8192-token,
 * 2048-wide shard needs 33 MiB).  All calls on one device share the array:
 * calls that overlap on one device (different streams, or different host
 * threads) race; calls on one stream are ordered. */
int tp_mlp_bwd_noalloc(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size,
                       const void* X, const void* W1_shard, int64_t ldw1, const void* W2_shard,
                       const void* H_save, const void* A_save, const void* dZ, float* dX_partial,
                       float* dW1_shard, float* db1_shard, float* dW2_shard);

/* Size in bytes of the static scratch array of tp_mlp_bwd_noalloc. */
size_t tpmlp_noalloc_scratch_bytes(void);

/* Backward of one column shard Y_i = X W_i (+ b_i) with no activation (the
 * QKV projection), dY_i the gradient of Y_i [wangyu 按列切分, backward]:
 *   dX_partial [T, K] fp32, lddx >= K   dY_i W_i^T (sum over shards = dX)
 *   dW_shard   [K, N/tp] fp32, lddw     X^T dY_i
 *   db_shard   [N/tp] fp32 or NULL      column sums of dY_i
 * X [T, K] (ldx), W_shard [K, N/tp] (ldw), dY [T, N/tp] (lddy), storage dtype. */
int column_parallel_bwd(void* stream, int dtype, int64_t T, int64_t K, int64_t N, int tp_size,
                        const void* X, int64_t ldx, const void* W_shard, int64_t ldw,
                        const void* dY, int64_t lddy, float* dX_partial, int64_t lddx,
                        float* dW_shard, int64_t lddw, float* db_shard);

/* Backward of one row shard Z_i = X_i W_i (the output projection) for the
 * full upstream gradient dY [T, N], which every shard receives unchanged
 * [wangyu 按行切分, backward]:
 *   dX_shard   [T, K/tp] fp32, lddx     dY W_i^T: column block i of dX
 *   dW_shard   [K/tp, N] fp32, lddw     X_i^T dY
 * X_shard [T, K/tp] (ldx), W_shard [K/tp, N] (ldw), dY (lddy), storage dtype. */
int row_parallel_bwd(void* stream, int dtype, int64_t T, int64_t K, int64_t N, int tp_size,
                     const void* X_shard, int64_t ldx, const void* W_shard, int64_t ldw,
                     const void* dY, int64_t lddy, float* dX_shard, int64_t lddx,
                     float* dW_shard, int64_t lddw);

/* ---- Gated MLP (SwiGLU) -------------------------------------------------
 * The Qwen3 MLP on [wangyu 多层感知机（MLP）中的张量并行]: gate = X W_gate,
 * up = X W_up, x = silu(gate) * up, down = x W_down, with W_gate and W_up
 * joined along their columns so one product yields both, the joined layer
 * split by columns and W_down by rows; silu(g) = g / (1 + exp(-g)); no
 * biases.  Shard i owns columns [i*Fs, (i+1)*Fs) of both W_gate and W_up,
 * Fs = F / tp_size, which must be a multiple of 8.
 *
 * Packed order: shard i's joined weight W_gu_shard [h, 2 Fs] holds in packed
 * column 16q + r the gate column 8q + r (r < 8) or the up column 8q + r - 8
 * (r >= 8) of the shard.  The saved pre-activations GU_save [T, 2 Fs] and the
 * gradient dW_gu_shard [h, 2 Fs] use the same order.  The bf16 GEMMs are the
 * only implementation (TPMLP_E_DTYPE for fp32).  */

/* Builds W_gu_shard [h, 2 Fs] (contiguous, storage dtype) from columns
 * [shard*Fs, (shard+1)*Fs) of W_gate [h, F] (ldg) and W_up [h, F] (ldu). */
int swiglu_pack_shard(void* stream, int dtype, int64_t h, int64_t F, int tp_size, int shard,
                      const void* W_gate, int64_t ldg, const void* W_up, int64_t ldu, void* W_gu_shard);

/* Writes the packed fp32 gradient dW_gu_shard [h, 2 Fs] into columns
 * [shard*Fs, (shard+1)*Fs) of dW_gate [h, F] (ldg) and dW_up [h, F] (ldu). */
int swiglu_unpack_grad(void* stream, int64_t h, int64_t F, int tp_size, int shard,
                       const float* dW_gu_shard, float* dW_gate, int64_t ldg, float* dW_up, int64_t ldu);

/* One shard's forward: GU = X W_gu_shard (packed), A = silu(gate) * up,
 * Z_partial = A W_down_shard.
 *   X             [T, h] bf16 (ld h)
 *   W_gu_shard    [h, 2 Fs] bf16, packed order
 *   W_down_shard  [Fs, h] bf16: rows i*Fs.. of W_down [F, h]
 *   GU_save       [T, 2 Fs] bf16 packed pre-activations, or NULL
 *   A_save        [T, Fs] bf16 (ld Fs)
 *   Z_partial     [T, h] fp32: this shard's partial of down */
int tp_swiglu_fwd(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size,
                  const void* X, const void* W_gu_shard, const void* W_down_shard,
                  void* GU_save, void* A_save, float* Z_partial);

/* Bytes of device workspace tp_swiglu_bwd needs (0 on bad args). */
size_t tp_swiglu_bwd_workspace_bytes(int dtype, int64_t T, int64_t h, int64_t F, int tp_size);

/* One shard's backward for the upstream gradient dZ [T, h] (bf16) of down.
 * With dA = dZ W_down_shard^T and, per column, dgate = dA * up * silu'(gate),
 * dup = dA * silu(gate) (packed as dGU, bf16, kept in the workspace):
 *   dX_partial     [T, h] fp32      dGU W_gu_shard^T (sum over shards = dX)
 *   dW_gu_shard    [h, 2 Fs] fp32   X^T dGU, packed order
 *   dW_down_shard  [Fs, h] fp32     A^T dZ
 * GU_save and A_save come from tp_swiglu_fwd.  workspace: device memory of at
 * least tp_swiglu_bwd_workspace_bytes() bytes, 256-byte aligned, owned by the
 * caller.  T = 0 writes zero weight gradients. */
int tp_swiglu_bwd(void* stream, int dtype, int64_t T, int64_t h, int64_t F, int tp_size,
                  const void* X, const void* W_gu_shard, const void* W_down_shard,
                  const void* GU_save, const void* A_save, const void* dZ,
                  float* dX_partial, float* dW_gu_shard, float* dW_down_shard,
                  void* workspace, size_t workspace_bytes);

/* ---- Sequence-parallel region (SP) ---------------------------------------
 * With SP the activations outside the tensor-parallel block — LayerNorm,
 * Dropout, the residual add — are split along the sequence: each GPU holds
 * rows [row0, row0 + rows) of the [T, h] residual stream; the block's input
 * is all-gathered and its output reduce-scattered [zouht 2.2.2 与序列并行结合,
 * 2.3 代价 (g / g*); sunjinbo SP · 序列并行].  On one GPU the gather is this
 * GPU's LayerNorm writing its rows of the gathered [T, h] buffer (pass Y =
 * gathered + row0*ldy) and the scatter is the sum of the shard partials over
 * its rows, fused below with the dropout and the residual.  Widths h must be
 * multiples of 8 and at most 16384; activations are bf16, LayerNorm
 * parameters, statistics and gradients fp32.
 *
 * Dropout keeps element (r, c) of the [T, h] tensor (r the global row) iff
 * word e % 4 (e = r*h + c) of Philox4x32-10 (Salmon et al., SC 2011) at
 * counter (n mod 2^32, n >> 32, 0, 0), n = e / 4, key (seed mod 2^32,
 * seed >> 32), is >= floor(p * 2^32); kept values are scaled by 1/(1-p).
 * The mask depends on the global row only, not on how rows are split.
 * 0 <= p < 1, else TPMLP_E_VALUE. */

/* Y = gamma * (X - mean) / sqrt(var + eps) + beta per row (biased variance).
 *   X [rows, h] bf16 (ldx); gamma, beta [h] fp32; Y [rows, h] bf16 (ldy);
 *   mean, rstd [rows] fp32: the row statistics the backward needs.
 * eps > 0, else TPMLP_E_VALUE. */
int layernorm_fwd(void* stream, int64_t rows, int64_t h, const void* X, int64_t ldx, const float* gamma,
                  const float* beta, float eps, void* Y, int64_t ldy, float* mean, float* rstd);

/* LayerNorm backward for upstream dY [rows, h] fp32 (lddy):
 *   dX [rows, h] fp32 (lddx) = rstd (g - mean(g) - xhat mean(g xhat)), g = dY gamma,
 *                              plus dRes [rows, h] bf16 (ldr) if not NULL
 *                              (the residual path's gradient);
 *   dgamma, dbeta [h] fp32 or NULL: sums over these rows of dY xhat and dY
 *   (this GPU's share; the full gradients sum over all GPUs' rows).
 * X, gamma, mean and rstd as given to / returned by layernorm_fwd. */
int layernorm_bwd(void* stream, int64_t rows, int64_t h, const void* X, int64_t ldx, const float* gamma,
                  const float* mean, const float* rstd, const float* dY, int64_t lddy, const void* dRes,
                  int64_t ldr, float* dX, int64_t lddx, float* dgamma, float* dbeta);

/* out = residual + Dropout(sum over s < tp_size of partials[s]) on this GPU's
 * rows: the reduce-scatter end of the block (shards added in ascending order
 * in fp32), then the sequence-split dropout and residual add, rounded once.
 *   partials   element (s, r, c) at partials[s*shard_stride + r*ldp + c], fp32
 *              (pass the pointer to this GPU's first row)
 *   residual   [rows, h] bf16 (ldr); out [rows, h] bf16 (ldo)
 *   row0       global row of the first row (selects the dropout bits) */
int sp_partial_sum_dropout_residual(void* stream, int tp_size, int64_t rows, int64_t h, const float* partials,
                                    int64_t shard_stride, int64_t ldp, const void* residual, int64_t ldr,
                                    float p, uint64_t seed, int64_t row0, void* out, int64_t ldo);

/* Backward of the dropout for this GPU's rows: dZ = kept ? dOut/(1-p) : 0,
 * dOut, dZ [rows, h] bf16.  Point dZ at this GPU's rows of the gathered
 * [T, h] upstream gradient of the tensor-parallel block (the all-gather). */
int sp_dropout_bwd(void* stream, int64_t rows, int64_t h, const void* dOut, int64_t ldi, float p, uint64_t seed,
                   int64_t row0, void* dZ, int64_t ldz);

/* ---- Attention core -------------------------------------------------------
 * Between the head-sharded QKV (column) and O (row) projections each shard
 * computes its own heads independently [csdn 1.2.2; zouht 2.2.1 多头注意力机制;
 * wangyu 注意力机制中的张量并行]: per head and sequence
 * O = softmax(Q K^T * scale) V (scale > 0, finite), with keys j > i masked
 * for query i when causal = 1.  T = batch * seq token rows (sequence b is rows
 * [b*seq, (b+1)*seq)); head h reads columns [h*head_dim, (h+1)*head_dim) of
 * Q, K, V (bf16, row strides ldq, ldk, ldv — e.g. the three blocks of the
 * fused QKV output, ld = 3*heads*head_dim) and writes the same columns of O
 * (bf16, ldo).  head_dim must be 128.  lse [heads, T] fp32 (row h*T + t)
 * receives log(sum_j exp(s_tj)) of each query row, or pass NULL.
 * workspace: device memory of at least attn_fwd_workspace_bytes() bytes,
 * 256-byte aligned, owned by the caller; causal calls on sequences longer
 * than 2048 keep per-chunk partial results there (the key range of a query
 * block is split over several workgroups and merged by log-sum-exp).  It may
 * be NULL (with workspace_bytes 0) when that size is 0 or causal = 0. */
int attn_fwd(void* stream, int64_t batch, int64_t seq, int heads, int head_dim, int causal, float scale,
             const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V, int64_t ldv, void* O,
             int64_t ldo, float* lse, void* workspace, size_t workspace_bytes);

/* Bytes of device workspace a causal attn_fwd needs (0 on bad args, and for
 * sequences of at most 2048): fp32 partial O tiles of 64 KB plus 512 bytes
 * of row log-sum-exp per work item (1.5 per query block of 128 rows, per
 * head and sequence, at 4096 tokens; at most 8 chunks per block). */
size_t attn_fwd_workspace_bytes(int64_t batch, int64_t seq, int heads);

/* Bytes of device workspace attn_bwd needs (0 on bad args): two fp32
 * [heads, T] arrays (the row sums D and the log-sum-exp in base 2) and, for
 * causal sequences longer than 2048, fp32 partial dQ tiles
 * of 64 KB, one per work item of the query blocks whose keys are split into
 * chunks (at most 8 chunks per block; about 4.5 tiles per query block of 128
 * rows, per head and sequence, at 32K tokens). */
size_t attn_bwd_workspace_bytes(int64_t batch, int64_t seq, int heads);

/* Backward of attn_fwd for the upstream gradient dO (bf16, same layout as O).
 * With P = softmax(Q K^T * scale) (recomputed from lse), D = rowsum(dO * O):
 *   dV = P^T dO, dS = P * (dO V^T - D), dQ = dS K * scale, dK = dS^T Q * scale,
 * written as bf16 into dQ, dK, dV (head h in columns [h*128, (h+1)*128), row
 * strides lddq, lddk, lddv — e.g. the three blocks of a fused dQKV buffer).
 * O and lse as written by attn_fwd.  Deterministic: no atomics.  workspace:
 * device memory of at least attn_bwd_workspace_bytes() bytes, 256-byte
 * aligned, owned by the caller. */
int attn_bwd(void* stream, int64_t batch, int64_t seq, int heads, int head_dim, int causal, float scale,
             const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V, int64_t ldv, const void* O,
             int64_t ldo, const void* dO, int64_t lddo, const float* lse, void* dQ, int64_t lddq, void* dK,
             int64_t lddk, void* dV, int64_t lddv, void* workspace, size_t workspace_bytes);

/* ---- Head-sharded attention block ----------------------------------------
 * One shard of the attention block whose heads are split over tp_size GPUs
 * [csdn 1.2.2 Self-Attention 模块的张量并行; zouht 2.2.1 多头注意力机制;
 * wangyu 注意力机制中的张量并行]: shard i owns heads [i*H/tp, (i+1)*H/tp),
 * i.e. columns c = [i*w, (i+1)*w), w = H/tp * head_dim, of each of the
 * projections Wq, Wk, Wv (a column split) and rows c of Wo (a row split); the
 * block output is the sum over shards of Z_i = O_i Wo[c, :].  No biases, bf16
 * storage, fp32 accumulation, head_dim 128, heads % tp_size == 0.
 *   X            [T, h] (ld h), T = batch * seq token rows
 *   Wqkv_shard   [h, 3w] (ld 3w) = [Wq[:, c] | Wk[:, c] | Wv[:, c]]
 *   Wo_shard     [w, h] (ld h) = Wo[c, :]
 *   QKV_save     [T, 3w] (ld 3w) bf16: X Wqkv_shard, kept for the backward
 *   O_save       [T, w] (ld w) bf16: the attention output of the shard's heads
 *   lse          [H/tp, T] fp32: log-sum-exp of each query row (as attn_fwd)
 *   Z_partial    [T, h] fp32 (ld h): this shard's partial of the output
 * causal and scale as in attn_fwd; workspace as attn_fwd's for the shard's
 * H/tp heads, at least tp_attn_fwd_workspace_bytes() bytes (checked before
 * anything is launched). */
int tp_attn_fwd(void* stream, int64_t batch, int64_t seq, int64_t h, int heads, int head_dim, int tp_size,
                int causal, float scale, const void* X, const void* Wqkv_shard, const void* Wo_shard,
                void* QKV_save, void* O_save, float* lse, float* Z_partial, void* workspace,
                size_t workspace_bytes);

/* Bytes of device workspace tp_attn_fwd needs (0 on bad args or when none). */
size_t tp_attn_fwd_workspace_bytes(int64_t batch, int64_t seq, int heads, int head_dim, int tp_size);

/* Bytes of device workspace tp_attn_bwd needs (0 on bad args). */
size_t tp_attn_bwd_workspace_bytes(int64_t batch, int64_t seq, int heads, int head_dim, int tp_size);

/* Backward of tp_attn_fwd for the gradient dZ [T, h] (bf16, ld h) of the
 * block output, which every shard receives whole [wangyu 按行切分, backward]:
 * dO = dZ Wo_shard^T, dWo_shard = O^T dZ, the attention backward gives dQKV,
 * dWqkv_shard = X^T dQKV and dX_partial = dQKV Wqkv_shard^T (the sum over
 * shards is dX [wangyu 按列切分, backward]).
 *   dX_partial   [T, h] fp32 (ld h)
 *   dWqkv_shard  [h, 3w] fp32 (ld 3w), the packed order of Wqkv_shard
 *   dWo_shard    [w, h] fp32 (ld h)
 * X, the weights, QKV_save, O_save and lse as passed to / written by
 * tp_attn_fwd.  workspace: at least tp_attn_bwd_workspace_bytes() bytes,
 * 256-byte aligned, owned by the caller (holds dO, dQKV in bf16 and the
 * attention backward's row sums). */
int tp_attn_bwd(void* stream, int64_t batch, int64_t seq, int64_t h, int heads, int head_dim, int tp_size,
                int causal, float scale, const void* X, const void* Wqkv_shard, const void* Wo_shard,
                const void* QKV_save, const void* O_save, const float* lse, const void* dZ, float* dX_partial,
                float* dWqkv_shard, float* dWo_shard, void* workspace, size_t workspace_bytes);

/* Status name, and the calling thread's message for its last non-OK status. */
const char* tpmlp_status_string(int status);
const char* tpmlp_last_error(void);

/* Library version string. */
const char* tpmlp_version(void);

/* Per-kernel timing on the launch stream (a profiling aid for benchmarks).
 * tpmlp_profile_enable(filter): while enabled, every kernel the library
 * launches whose role name contains `filter` ("" = all, NULL = disable) is
 * bracketed by two hipEvents recorded on the launch stream.  A launch that
 * runs several products reports their role names joined by '+'.
 * tpmlp_profile_collect(buf, len): waits for the recorded events, writes the
 * launches in order as a JSON list [["role", "kernel_symbol", ms, ghz], ...]
 * to buf and clears the record.  ghz is the shader clock over workgroup 0's
 * main loop for bf16 GEMM launches (sampled with the s_memtime and
 * s_memrealtime counters; the first tpmlp_profile_enable allocates a small
 * device buffer for these samples, kept until the process ends), -1 for
 * other kernels.  Returns TPMLP_OK, TPMLP_E_SHAPE if the text did not
 * fit in len bytes (it is truncated), or TPMLP_E_HIP. */
int tpmlp_profile_enable(const char* filter);
int tpmlp_profile_collect(char* buf, size_t len);

#ifdef __cplusplus
}
#endif
#endif /* TPMLP_H */
