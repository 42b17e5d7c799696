/*
 * fa.h -- C ABI of the exact, IO-aware attention library for AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention
 *     S = scale * Q K^T,  P = softmax(S) row-wise,  O = P V
 * tile by tile with an online softmax, so that S and P never reach device
 * memory; it writes only O and one log-sum-exp per row.  The backward pass
 * recomputes each P tile from that log-sum-exp and uses
 * delta_i = rowsum(dO_i o O_i) to form dQ, dK and dV.
 *
 * Sources for what is computed:
 *  - "FlashAttention-1: eliminating IO" (deep-learning-notes ch10.2):
 *    section 10.2.1 (definition and safe softmax), section 10.2.2 (online
 *    rescaling with alpha = exp(m_old - m_new)), section 10.2.3 (forward,
 *    scale 1/sqrt(d)), section 10.2.4 (recompute backward, dS = P o (dP - delta),
 *    delta_i = dO_i . O_i), section 10.2.5 (one workgroup per query block).
 *  - "Flash Attention V1/V2/V3" explainer: V2 section (query-block work
 *    partitioning, deferred normalisation, mask fused into the score stage) and
 *    V3 section (FP8 inputs with FP32 accumulation and scaling factors).
 *  - "5.4 FlashAttention (1/2/3)" reading notes, code 3-1 (running max,
 *    alpha, unnormalised accumulator, one final division).
 *
 * Conventions shared by every entry point
 *  - Tensors Q, K, V, O, dO, dQ, dK, dV are contiguous row-major [B, H, N, d]
 *    arrays (d innermost).  LSE and delta are contiguous [B, H, N] float32.
 *  - Causal: key j is visible to query i iff j <= i (square attention).
 *  - LSE_i = ln sum_j exp(S_ij) in the natural log of the scaled scores.
 *  - All pointers are device pointers the caller owns.  The library allocates
 *    nothing and never synchronises: work is enqueued on `stream` (a
 *    hipStream_t; NULL = the default stream) and the call returns.  Calls on
 *    different streams are independent.  The only mutable global state is the
 *    per-device scratch of fa_bwd_noalloc (see there).
 *  - Supported head sizes d: 64 and 128.  Any N >= 1 (a head's K or V may
 *    exceed 4 GiB); B * H * N == 0 is a no-op returning FA_OK.  Tensor
 *    pointers must be 16-byte aligned, LSE and workspace 4-byte aligned.
 *    B*H*N*d must stay below 2^40 elements.
 *  - scale must be finite and > 0.
 *  - Errors: argument problems return FA_ERR_INVALID_ARG or FA_ERR_UNSUPPORTED
 *    before anything is launched; a failed launch returns FA_ERR_HIP.  No
 *    exception or abort crosses the ABI.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats.  FA_FP8_E4M3 is OCP float8 e4m3fn (bias 7, no infinity,
 * max finite 448), the format gfx950's matrix cores take. */
typedef enum { FA_FP32 = 0, FA_BF16 = 1, FA_FP8_E4M3 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad scale, bad flag */
  FA_ERR_UNSUPPORTED = 2, /* valid but not provided: d not in {64,128}, fp8 backward */
  FA_ERR_HIP = 3          /* the HIP runtime rejected a launch */
} fa_status;

/* Forward pass ("FlashAttention-1: eliminating IO", sections 10.2.1-10.2.3;
 * explainer V2 and V3 sections).
 *   q, k, v : [B,H,N,d] inputs of type `dtype` (fp8: e4m3fn codes, 1 byte each)
 *   o       : [B,H,N,d] output; float32 for FA_FP32, bfloat16 for FA_BF16 and
 *             for FA_FP8_E4M3
 *   lse     : [B,H,N] float32 output, ln sum_j exp(S_ij) over visible keys
 *   scale   : multiplies Q K^T (1/sqrt(d) on the pages)
 *   causal  : 0 or 1
 *   q_descale, k_descale, v_descale : fp8 only -- the real value of a code c
 *             is decode(c) * descale (one scale per tensor, finite, > 0);
 *             ignored for the other formats.
 * Accumulation is float32 for every format.
 * Schedule (bf16, d = 128, no bias; read from the environment variable
 * FA_FWD_SCHEDULE on every fa_fwd and fa_fwd_bias call): unset, empty or
 * "interleaved" -- the default, each wave weaves a tile's softmax into the
 * next tile's matrix products; "pingpong" -- two wave groups per SIMD
 * alternate products and softmax (the reading notes' three-generation table,
 * FA3 ping-pong scheduling); "rows64" -- 64 query rows per wave, one wave per
 * SIMD.  All three compute the same outputs up to rounding (their float32
 * additions run in different orders); any other
 * value returns FA_ERR_INVALID_ARG. */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, int dtype, float q_descale,
                 float k_descale, float v_descale, void* stream);

/* Forward pass on fp8 e4m3fn inputs with microscaling block scales (the
 * finer-grained scale management the explainer's V3 section names for FP8;
 * per-tensor scales, fa_fwd with FA_FP8_E4M3, are the coarse case).  Each
 * block of 32 consecutive elements along a product's contraction shares one
 * power-of-two scale stored as an e8m0 byte E (value 2^(E - 127); E = 255 is
 * not accepted by the hardware and must not occur):
 *   q_scale, k_scale : [B,H,N,4] bytes -- byte c (c < d/32) of row n scales
 *                      head dims 32c .. 32c+31 (the contraction of Q K^T);
 *                      one 4-byte word per row whatever d, the rest unused
 *   v_scale          : [B,H,ceil(N/32),d] bytes -- block b of head dim j
 *                      covers keys 32b .. 32b+31 (the contraction of P V)
 * The real value of a code is decode(code) * 2^(E - 127) of its block.  The
 * other arguments are those of fa_fwd (o is bfloat16, lse float32); q, k, v,
 * o need 16-byte alignment, the scale arrays 4-byte alignment.  Same status
 * codes; nothing is launched on an error. */
fa_status fa_fwd_mxfp8(const void* q, const void* k, const void* v, const void* q_scale,
                       const void* k_scale, const void* v_scale, void* o, float* lse, int B,
                       int H, int N, int d, float scale, int causal, void* stream);

/* Forward pass with an additive bias on the scaled scores: the explainer's
 * V2 section merges mask and bias into the score computation.
 *   s_ij = scale * q_i . k_j + bias[b][h][i][j]
 * then the softmax over the visible keys (all, or j <= i with causal = 1).
 * A bias of -INFINITY masks a key, so general masks are biases of 0 and -inf
 * (key padding, sliding windows, block patterns ...).  Bias values must be
 * finite or -inf.  A row whose visible scores are all -inf has an empty
 * softmax: its output row is 0 and its LSE is -inf.
 *   bias   : float32, element (b, h, i, j) at
 *            bias[b*bias_stride_b + h*bias_stride_h + i*bias_stride_q + j];
 *            strides in elements, each a non-negative multiple of 4 (0
 *            broadcasts: a [1,1,N,N] bias has strides 0, 0, row pitch; a
 *            per-key [B,1,1,N] padding mask has strides pitch, 0, 0).  The
 *            pointer is 16-byte aligned and the caller owns the buffer.  One
 *            (b, h) slice, (N-1)*bias_stride_q + N elements, must stay below
 *            2^30 - 1024 elements.  NULL means no bias (exactly fa_fwd).
 * dtype: FA_FP32 or FA_BF16 (FA_FP8_E4M3 returns FA_ERR_UNSUPPORTED).  The
 * other arguments are those of fa_fwd.  Same status codes; nothing is
 * launched on an error. */
fa_status fa_fwd_bias(const void* q, const void* k, const void* v, const float* bias,
                      long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                      void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
                      int dtype, void* stream);

/* Standard attention, the baseline the pages measure the IO-aware method
 * against (reading notes "5.4 FlashAttention (1/2/3)", standard attention;
 * explainer, background section): S = scale Q K^T is written to device
 * memory in float32, a row-wise softmax reads it and writes P in bfloat16,
 * and O = P V reads P back -- O(N^2) bytes of device-memory traffic per head
 * where fa_fwd moves O(N d).  Same result as fa_fwd up to rounding (P is
 * normalised before the product), for measuring that difference; it is not
 * an alternative implementation of the library's path.
 *   q, k, v, o, lse, scale, causal : as fa_fwd; dtype must be FA_BF16
 *             (FA_FP32 and FA_FP8_E4M3 return FA_ERR_UNSUPPORTED)
 *   workspace : 256-byte aligned device buffer of at least
 *             fa_std_workspace_size() bytes; on return it holds S
 *             ([B,H,N,ldp] float32, ldp = N rounded up to 64) followed (at
 *             the next 256-byte boundary) by P ([B,H,N,ldp] bfloat16, zero
 *             where masked and in the padding)
 * B*H must stay below 65536 and N below 2^22 (FA_ERR_UNSUPPORTED). */
size_t fa_std_workspace_size(int B, int H, int N, int d);
fa_status fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                     float scale, int causal, int dtype, void* stream);

/* Bytes of device workspace fa_bwd needs for these sizes: delta_i =
 * dO_i . O_i of "FlashAttention-1: eliminating IO", section 10.2.4, one
 * float32 per row at the start of the workspace, rounded up to 256 bytes.
 * Returns 0 for invalid sizes (nothing is checked beyond the sizes). */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/* Backward pass ("FlashAttention-1: eliminating IO", section 10.2.4).
 *   q, k, v, o, dout : [B,H,N,d] of type `dtype` (o as written by fa_fwd)
 *   lse              : [B,H,N] float32 from fa_fwd
 *   dq, dk, dv       : [B,H,N,d] outputs of type `dtype`
 *   workspace        : device buffer of at least fa_bwd_workspace_size() bytes;
 *                      on return its first B*H*N floats hold
 *                      delta_i = sum_c dO_ic O_ic
 *   workspace_bytes  : its size, checked
 * dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO with dS = P o (dP - delta).
 * Supported dtypes: FA_FP32 and FA_BF16 (FA_FP8_E4M3 -> FA_ERR_UNSUPPORTED). */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                 int dtype, void* stream);

/* The backward's stages, with fa_bwd's arguments and validation (each stage
 * uses the pointers it needs; the others must still be valid).  They let a
 * caller schedule or time the stages separately.
 *   fa_bwd_delta : delta_i = dO_i . O_i into the workspace (FA1 page, 10.2.4)
 *   fa_bwd_dq    : dQ.  FA_BF16: it also forms delta from O and dO itself and
 *                  writes it into the workspace; FA_FP32: it reads delta from
 *                  the workspace
 *   fa_bwd_dkdv  : dK and dV, reading delta from the workspace
 * fa_bwd(...) is exactly, on one stream, fa_bwd_dq(...); fa_bwd_dkdv(...) for
 * FA_BF16 and fa_bwd_delta(...); fa_bwd_dkdv(...); fa_bwd_dq(...) for FA_FP32.
 * A stage that reads delta needs it written earlier on the same stream (or
 * made visible by the caller's synchronisation). */
fa_status fa_bwd_delta(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                       float scale, int causal, int dtype, void* stream);
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                      float scale, int causal, int dtype, void* stream);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                    int dtype, void* stream);

/* Backward pass with the additive bias of fa_fwd_bias: P is recomputed as
 * exp(scale q.k + bias - LSE) from the LSE that fa_fwd_bias wrote (rows with
 * LSE = -inf have P = 0 and add nothing).  The bias is an input: no gradient
 * is formed for it.  Arguments as fa_bwd plus the bias of fa_fwd_bias;
 * enqueues the same stages as fa_bwd.  FA_FP8_E4M3 returns
 * FA_ERR_UNSUPPORTED. */
fa_status fa_bwd_bias(const void* q, const void* k, const void* v, const float* bias,
                      long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk,
                      void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N,
                      int d, float scale, int causal, int dtype, void* stream);

/* Largest B * H * N that fa_bwd_noalloc accepts: its delta scratch holds one
 * float32 per row, 16 MiB per GPU. */
#define FA_NOALLOC_MAX_ROWS (1 << 22)

/* fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same computation, kernels and outputs as fa_bwd
 * (bitwise), same arguments minus workspace and workspace_bytes.  delta lives
 * in a device-global array of FA_NOALLOC_MAX_ROWS floats that the library
 * image holds on each GPU it runs on until the process ends; its contents
 * after a call are that call's delta.
 *  - B * H * N > FA_NOALLOC_MAX_ROWS returns FA_ERR_UNSUPPORTED (nothing is
 *    launched); the other argument errors are fa_bwd's.
 *  - The current device must be the device of `stream` (FA_ERR_INVALID_ARG
 *    otherwise).  The first call on a device looks the array's address up in
 *    the runtime (no allocation by this library); make that first call
 *    outside stream capture.
 *  - All calls on one GPU share the array: calls that overlap in time on one
 *    GPU (different streams without ordering, or several host threads) race
 *    on it and give undefined results.  Calls ordered on one stream are
 *    safe.  Nothing in the array needs clearing: every call writes delta
 *    before reading it. */
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int H, int N, int d, float scale, int causal, int dtype, void* stream);

/* Static, NUL-terminated description of a status code (never NULL).  The
 * pages define no error convention; the codes are this library's own. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
