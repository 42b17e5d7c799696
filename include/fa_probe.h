/* fa_probe.h -- C ABI of libfa_probe.so: a matrix-core rate probe for MI355X
 * (gfx950).  A measurement aid, not part of attention: bench.py and the tests
 * read the attention kernels' rates against what it measures, beside the
 * published peak.  Separate from libfa.so (include/fa.h), which holds only
 * attention.
 *
 * Callers: benchmarks and tests that need the rate the matrix cores sustain
 * on realistic operand bits at the clock the chip settles to within its
 * power budget.
 */
#ifndef FA_PROBE_H_
#define FA_PROBE_H_

#ifdef __cplusplus
extern "C" {
#endif

/* Element types and status codes: the same values as FA_BF16 / FA_FP8_E4M3 /
 * FA_FP32 and fa_status in fa.h, so callers of both libraries use one set. */
enum { FA_PROBE_FP32 = 0, FA_PROBE_BF16 = 1, FA_PROBE_FP8_E4M3 = 2 };
enum {
  FA_PROBE_OK = 0,
  FA_PROBE_ERR_INVALID_ARG = 1,
  FA_PROBE_ERR_UNSUPPORTED = 2,
  FA_PROBE_ERR_HIP = 3
};

/* Enqueues a pure stream of 32x32 matrix-core products (bf16 32x32x16 or fp8
 * 32x32x64: 32768 or 131072 FLOPs per product) on fixed pseudo-random
 * per-lane operands on `stream` (a hipStream_t; NULL: the null stream):
 * `blocks` workgroups of 512 threads (two waves per SIMD; use a multiple of
 * the CU count), each thread running iters * 8 products.  Every thread writes
 * one float to out[block * 512 + thread]: `out` is caller-owned device memory
 * of blocks * 512 floats, 4-byte aligned.  Timing the launch gives the rate;
 * total FLOPs = blocks * 8 waves * iters * 8 * (FLOPs per product).
 * dtype FA_PROBE_BF16 or FA_PROBE_FP8_E4M3 (FA_PROBE_FP32:
 * FA_PROBE_ERR_UNSUPPORTED, anything else FA_PROBE_ERR_INVALID_ARG); blocks
 * 1..65536, iters 1..2^20, out non-NULL and aligned, else
 * FA_PROBE_ERR_INVALID_ARG before any launch; FA_PROBE_ERR_HIP if the launch
 * fails.  Returns without waiting for the kernel. */
int fa_measure_mfma_rate(float* out, int blocks, int iters, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */
