/* Machine probes (libtpmlp_probe.so): measurements of the hardware limits the
 * GEMM kernels are designed against.  They compute nothing of the MLP block
 * and are not part of libtpmlp.so; `python3 bench.py --probe` runs them.
 *
 * Each call allocates and frees its own device buffers (hipMalloc/hipFree),
 * launches on the null stream of the current device and synchronises before
 * it returns.  Return value: 0 on success; 2 for bad arguments, 3 when an
 * address the launch would form falls outside its buffer (checked on the
 * host before any launch), 1 for a HIP error; tpmlp_probe_last_error() then
 * holds a message. */
#ifndef TPMLP_PROBE_H
#define TPMLP_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Per-CU load path: 256 workgroups of 4 waves (one per CU) each load the
 * operand tiles of one 256x256 output tile (A: K-contiguous rows, lda >= 4096
 * bf16 per row, 8192 rows; B: N-contiguous K-rows, ldb >= 2048, 4096 rows)
 * for 64 K steps of 64 elements, 64 KB per CU per step.
 *   mode     0: LDS DMA (buffer_load_dwordx4 ... lds), one step of loads in
 *               flight beyond the one waited for;
 *            1: plain 16-byte loads into registers, two steps in flight;
 *            2: as 1, then written into a two-stage LDS ring (ds_write_b128,
 *               one barrier per step).
 *   pattern  0: each step half A (loads of 8 rows x 128 B), half B (2 K-rows
 *               x 512 B), as in the kernels; 1: A only; 2: B only; 3: A only
 *               with a load's 8 rows 32 rows apart.
 *   reps     timed launches (after 3 untimed ones).
 * out[0] microseconds per launch, out[1] shader clock in GHz (workgroup 0,
 * from the clock counters), out[2] GB/s over all CUs, out[3] bytes per clock
 * per CU. */
int tpmlp_probe_load_path(int mode, int pattern, int lda, int ldb, int reps, double* out);

/* LDS read rate: 256 workgroups (one per CU) of `waves` (4, 8 or 16) waves,
 * each issuing `iters` groups of 8 independent reads at conflict-free
 * addresses and waiting for each group.  transposing 0: ds_read_b128 (1 KB a
 * read); 1: ds_read_b64_tr_b16 (512 B).  out[0] shader clocks of workgroup 0,
 * out[1] bytes per clock per CU. */
int tpmlp_probe_lds_read(int transposing, int waves, int iters, double* out);

/* Message for the last non-zero return of a probe call (not thread-safe). */
const char* tpmlp_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPMLP_PROBE_H */
