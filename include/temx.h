/*
 * temx.h -- C ABI of the MXFP8 Linear hot path for AMD Instinct MI355X (gfx950).
 *
 * The library computes the FP8 Linear path that sits behind Transformer
 * Engine's Linear / LayerNormMLP modules on ROCm:
 *   - per-tensor amax (two-stage, no atomics) and the current-scaling cast;
 *   - MXFP8 1-D block quantization of bf16 tensors, rowwise and transposed
 *     columnwise (32-element blocks, one E8M0 power-of-two scale per block),
 *     and the fused cast-transpose with bias gradient;
 *   - delayed scaling (amax history) and the per-tensor FP8 GEMM;
 *   - blockwise FP8 (1 x 128 / 128 x 128 blocks with FP32 scale inverses):
 *     quantization and the GEMM, with the scales cast to E8M0 or as FP32;
 *   - the MXFP8 x MXFP8 -> fp32-accumulate GEMM with bias, GELU(tanh) and
 *     GELU-aux (pre-activation) epilogues;
 *   - a single-launch grouped (MoE) variant over ragged expert row counts.
 *
 * Sources, cited by page title and section:
 *   [ROCm-TE]  "Transformer Engine On ROCm and AMDGPU" (ROCm/TransformerEngine
 *              README): "MXFP8 support on ROCm (gfx95x only)", "Blockwise FP8
 *              GEMM support on ROCm" (E8M0 power-of-two scales), "Two-stage
 *              amax Kernel", "Experimental Triton Kernels on ROCm"
 *              (cast_transpose, cast_transpose_bgrad), "Grouped GEMM using
 *              CK_Tile".
 *   [TE-JAX]   "Getting Started" (Transformer Engine JAX quickstart): GELU
 *              with the tanh approximation; "Enabling Quantization" (HYBRID).
 *   [FP8-WF]   "Workflow: NVIDIA TransformerEngine FP8 Training Quickstart",
 *              Step 4: E4M3 forward / E5M2 backward (HYBRID); current scaling.
 *   [HK-PR]    "HipKittens MXFP8 GEMM Support" (ROCm/TransformerEngine PR
 *              #566): description (BIAS, GELU AUX epilogues) and review
 *              threads (1-D MXFP8 scaling mode; K % 128, M % 16, N % 16;
 *              "TN" layout).
 *
 * Encoding conventions (the pages do not define them; OCP FP8 / OCP MX):
 *   E4M3 is the OCP "FN" variant (max 448, no Inf), E5M2 is IEEE-like (max
 *   57344).  Block scale code = max(biased_exp(block amax) - emax, 0) with
 *   emax 8 (E4M3) / 15 (E5M2), i.e. floor(log2(amax)) - emax biased by 127.
 *   Element codes are the saturating round-to-nearest-even encoding of
 *   x / 2^(code - 127); the sign is kept (negative underflow gives 0x80).
 *   Inputs holding NaN or Inf give unspecified codes.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless stated; the caller owns every
 *     buffer.  The library never allocates, frees or caches device memory
 *     and keeps no state between calls other than a per-device cache of the
 *     compute-unit count and of the architecture check.
 *   - All work is enqueued on `stream` (0 = the null stream); no entry point
 *     synchronizes the host.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     failure a non-TE_OK status is returned and nothing runs.  A call with
 *     work to enqueue then checks that the current device is a gfx950
 *     (looked up once per device and cached) and returns TE_ERR_ARCH
 *     otherwise.  A failed launch returns TE_ERR_HIP.  Nothing throws across
 *     the ABI.
 *   - Data pointers must be 16-byte aligned (TE_ERR_ALIGN otherwise); scale
 *     pointers and scalar outputs have no alignment requirement beyond
 *     their type.
 *   - Tensors are row-major.  bf16 values are passed as their uint16 bit
 *     patterns.  MXFP8 data is uint8 [rows, K] with E8M0 scales uint8
 *     [rows, K/32] (unpadded, row-major).
 */
#ifndef TEMX_H
#define TEMX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TE_OK = 0,
  TE_ERR_NULL = 1,       /* a required pointer is NULL, or an unused one is not */
  TE_ERR_SHAPE = 2,      /* a size violates the entry point's shape rules */
  TE_ERR_ALIGN = 3,      /* a data pointer is not 16-byte aligned */
  TE_ERR_DTYPE = 4,      /* unsupported format / dtype / format combination */
  TE_ERR_WORKSPACE = 5,  /* workspace smaller than the size query returns */
  TE_ERR_HIP = 6,        /* a HIP call or kernel launch failed */
  TE_ERR_VALUE = 7,      /* an enum argument is out of range */
  TE_ERR_ARCH = 8        /* the current device is not a gfx950 (the kernels are built for it only) */
} te_status;

typedef enum { TE_BF16 = 0, TE_FP32 = 1, TE_E4M3 = 2, TE_E5M2 = 3, TE_E8M0 = 4, TE_FP16 = 5 } te_dtype;

typedef enum {
  TE_EPI_NONE = 0,
  TE_EPI_BIAS = 1,
  TE_EPI_BIAS_GELU_AUX = 2,
  TE_EPI_DGELU = 3,      /* backward of BIAS_GELU_AUX: D = acc * gelu_tanh'(aux) */
  TE_EPI_ACCUMULATE = 4  /* fp32 D += acc */
} te_epilogue;

typedef enum { TE_ROWWISE = 1, TE_COLWISE = 2, TE_BOTH = 3 } te_qdir;

typedef enum { TE_AMAX_MAX = 0, TE_AMAX_MOST_RECENT = 1 } te_amax_algo;

/* How the blockwise FP8 GEMM applies its FP32 block scales. */
typedef enum {
  TE_BLOCK_SCALES_E8M0 = 0, /* cast to E8M0 (smallest power of two >= s) first: the gfx950 default */
  TE_BLOCK_SCALES_FP32 = 1  /* the FP32 scales themselves */
} te_block_scaling;

/* Human-readable name of a status code (static storage). */
const char* te_status_str(te_status status);

/*
 * Per-tensor amax, two-stage ([ROCm-TE] "Two-stage amax Kernel"): stage one
 * writes one partial maximum per workgroup into `workspace`, stage two
 * reduces them; no atomics.
 *   x          bf16 [n]; n >= 0 (n == 0 gives amax 0)
 *   amax_out   float [1], device: max |x_i| (exact; -0 counts as 0)
 *   workspace  device scratch of at least te_amax_workspace_size(n) bytes
 */
size_t te_amax_workspace_size(int64_t n);
te_status te_amax_reduce(const uint16_t* x, int64_t n, float* amax_out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Current-scaling FP8 cast ([FP8-WF] Step 4, Float8CurrentScaling; margin 0
 * as in the [TE-JAX] recipes): amax as above, then on the device
 *   scale     = fl32(fmt_max / amax)  (fmt_max 448 for E4M3, 57344 for E5M2;
 *               amax == 0 gives 1; a quotient beyond the float range gives
 *               the largest finite float)
 *   scale_inv = fl32(1 / scale)
 *   q_i       = saturating RNE encode of fl32(x_i * scale).
 *   x          bf16 [n]
 *   fmt        TE_E4M3 or TE_E5M2
 *   q_out      uint8 [n]
 *   amax_out, scale_out, scale_inv_out   float [1] each, device
 *   workspace  at least te_amax_workspace_size(n) bytes
 */
te_status te_fp8_cast_current_scaling(const uint16_t* x, int64_t n, te_dtype fmt, uint8_t* q_out,
                                      float* amax_out, float* scale_out, float* scale_inv_out,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The current-scaling cast above, allocating nothing and taking no
 * workspace: for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * stage-one partial maxima live in a static device array of the library
 * (2 KB: at most 512 partials, one per amax workgroup, which serves every
 * n the entry point accepts).  Each GPU holds its own copy from the first
 * call on it until the process ends; its address is looked up on that first
 * call with the device current.  Arguments, results and errors are those of
 * te_fp8_cast_current_scaling (minus the workspace); the results are
 * bit-identical to it.  Calls on one GPU share the array, so calls that
 * overlap in time on one GPU (different streams, or different host threads)
 * race and give unspecified results; calls in one stream are ordered and
 * safe.  Nothing in the array needs clearing between calls: each call
 * writes every entry it reads.
 */
te_status te_fp8_cast_current_scaling_noalloc(const uint16_t* x, int64_t n, te_dtype fmt, uint8_t* q_out,
                                              float* amax_out, float* scale_out, float* scale_inv_out,
                                              hipStream_t stream);

/*
 * Delayed-scaling FP8 cast ([TE-JAX] README example and "Enabling
 * Quantization": DelayedScaling with margin, interval, an amax history of
 * length 16 and the "max" algorithm; [FP8-WF] Step 4: a history window of
 * amax values).  One call is one step on a tensor:
 *   1. q_i = saturating RNE encode of fl32(x_i * scale), with the scale as it
 *      stands on entry; q_scale_inv_out = fl32(1 / that scale) (what a GEMM
 *      on q takes as its alpha factor);
 *   2. the tensor's amax enters amax_history, newest first (the oldest drops);
 *   3. r = max(amax_history) (TE_AMAX_MAX) or amax_history[0]
 *      (TE_AMAX_MOST_RECENT); if r is positive and finite,
 *      scale = fl32(fl32(fmt_max / r) / 2^margin) (a quotient beyond float
 *      gives the largest finite float), else scale is kept.
 *   x            bf16 [n]
 *   fmt          TE_E4M3 or TE_E5M2
 *   q_out        uint8 [n]
 *   q_scale_inv_out, scale (in/out)   float [1] each, device
 *   amax_history float [history_len], device, in/out; 1 <= history_len <= 1024
 *   margin       0 .. 64
 *   workspace    at least te_amax_workspace_size(n) bytes
 * Initial state: scale = 1, history all zeros.  How often the scale is
 * updated (the recipe's interval) is the caller's choice of when to call.
 */
te_status te_fp8_cast_delayed_scaling(const uint16_t* x, int64_t n, te_dtype fmt, uint8_t* q_out,
                                      float* q_scale_inv_out, float* scale, float* amax_history,
                                      int history_len, te_amax_algo algo, int margin,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * MXFP8 1-D block quantization ([ROCm-TE] "MXFP8 support on ROCm"; scales
 * E8M0 per [ROCm-TE] "Blockwise FP8 GEMM support"; HYBRID formats per
 * [FP8-WF] Step 4; the transposed copy is what cast_transpose provides in
 * [ROCm-TE] "Experimental Triton Kernels on ROCm").
 *   x       bf16 [rows, cols]
 *   fmt     TE_E4M3 or TE_E5M2
 *   dir     TE_ROWWISE, TE_COLWISE or TE_BOTH
 *   rowwise (dir & TE_ROWWISE): blocks of 32 along cols; needs cols % 32 == 0.
 *           q_row uint8 [rows, cols], s_row uint8 [rows, cols/32]
 *   colwise (dir & TE_COLWISE): blocks of 32 down each column, stored
 *           transposed; needs rows % 32 == 0 and cols % 8 == 0.
 *           q_col uint8 [cols, rows], s_col uint8 [cols, rows/32]
 *   Output pointers of a direction not requested must be NULL.
 *   TE_BOTH makes both copies in one pass (x is read once).
 *   rows, cols >= 0; an empty tensor enqueues nothing.
 */
te_status te_mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t cols, te_dtype fmt, te_qdir dir,
                            uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                            hipStream_t stream);

/*
 * Cast-transpose with bias gradient, the fused kernel that [ROCm-TE]
 * "Experimental Triton Kernels on ROCm" names cast_transpose_bgrad: one pass
 * over an output gradient x = dY [rows = tokens, cols = features] writes
 * both MXFP8 copies, exactly as te_mxfp8_quantize(dir = TE_BOTH), and
 *   bgrad[c] = sum over r of x[r, c]
 * (the gradient of the bias of the Linear whose output gradient is x),
 * accumulated in fp32 in a fixed order, so the result is deterministic.
 *   x           bf16 [rows, cols]; rows % 32 == 0 and cols % 32 == 0
 *   fmt         TE_E4M3 or TE_E5M2 (E5M2 for gradients in HYBRID)
 *   q_row, s_row, q_col, s_col   as te_mxfp8_quantize with TE_BOTH
 *   bgrad       [cols], bgrad_dtype TE_FP32 (float) or TE_BF16 (round to
 *               nearest even of the fp32 sum); aligned to its type
 *   workspace   device scratch of at least
 *               te_mxfp8_quantize_bgrad_workspace_size(rows, cols) bytes,
 *               4-byte aligned (fp32 partial sums per workgroup row tile)
 * rows == 0 writes zeros to bgrad; cols == 0 enqueues nothing.
 */
size_t te_mxfp8_quantize_bgrad_workspace_size(int64_t rows, int64_t cols);
te_status te_mxfp8_quantize_bgrad(const uint16_t* x, int64_t rows, int64_t cols, te_dtype fmt,
                                  uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                                  void* bgrad, te_dtype bgrad_dtype, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * MXFP8 GEMM, "TN" ([HK-PR] description and review threads):
 *   D[m, n] = epi( sum_k A[m, k] * B[n, k] )   with fp32 accumulation, where
 *   A[m, k] = val(a[m, k]) * 2^(a_scale[m, k/32] - 127) (likewise B).
 *   a        uint8 [M, K], a_scale uint8 [M, K/32], a_fmt E4M3 or E5M2
 *   b        uint8 [N, K], b_scale uint8 [N, K/32], b_fmt E4M3 or E5M2
 *            (E5M2 x E5M2 is rejected with TE_ERR_DTYPE)
 *   d        [M, N], d_dtype TE_BF16 (round to nearest even) or TE_FP32
 *   epi      TE_EPI_NONE:          D = acc
 *            TE_EPI_BIAS:          D = acc + bias[n]
 *            TE_EPI_BIAS_GELU_AUX: pre = acc + bias[n]; aux = bf16(pre);
 *                                  D = gelu_tanh(pre)  ([TE-JAX] tanh GELU)
 *            TE_EPI_DGELU:         D = acc * gelu_tanh'(aux[m, n]): the
 *                                  backward of BIAS_GELU_AUX, where aux is
 *                                  the pre-activation the forward saved
 *                                  (read here) and acc the gradient of the
 *                                  GELU output
 *            TE_EPI_ACCUMULATE:    D = D + acc with D fp32 (read and
 *                                  written; the weight gradient added into
 *                                  an fp32 main gradient, beta = 1)
 *   bias     bf16 [N]; required iff epi is BIAS or BIAS_GELU_AUX, NULL otherwise
 *   aux      bf16 [M, N]; required iff epi is BIAS_GELU_AUX (written) or
 *            DGELU (read), NULL otherwise
 *   TE_EPI_ACCUMULATE needs d_dtype == TE_FP32 (TE_ERR_DTYPE otherwise).
 *   Shapes: M, N, K >= 0; K % 128 == 0, M % 16 == 0, N % 16 == 0 (the
 *   [HK-PR] checks; M and N need not be multiples of the tile size);
 *   K <= 2^23 (the tile copies use 32-bit offsets), M, N < 2^31 - 256.
 *   M == 0 or N == 0 enqueues nothing; K == 0 gives D = epi(0).
 *   workspace: optional device scratch, owned by the caller and free for
 *   reuse once the GEMM has run (stream order).  te_mxfp8_gemm_workspace_size
 *   returns the bytes that enable the faster path for the shape on the
 *   current device, 0 where there is none: grids the 4-wave 256 x 256 tile
 *   serves (K % 1024 == 0, K >= 2048 and 32 or more K steps per CU) take
 *   (M + N) K / 32 bytes (A's part rounded up to 256)
 *   for a rearranged copy of both operands' E8M0 scales (blocks of 4 K steps,
 *   a tile row's 16 bytes contiguous), written by the GEMM itself on the same
 *   stream.  With a NULL workspace, a smaller one, one not 256-byte aligned,
 *   or scale arrays not 16-byte aligned, the GEMM runs without it (same
 *   results, bit for bit); a workspace is never an error.  Calls that share
 *   one workspace must be ordered on one stream.
 */
size_t te_mxfp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
te_status te_mxfp8_gemm(const uint8_t* a, const uint8_t* a_scale, te_dtype a_fmt,
                        const uint8_t* b, const uint8_t* b_scale, te_dtype b_fmt,
                        int64_t M, int64_t N, int64_t K,
                        void* d, te_dtype d_dtype, te_epilogue epi,
                        const uint16_t* bias, uint16_t* aux,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Per-tensor FP8 GEMM (the GEMM of the delayed and current scaling recipes):
 *   D = epi( a_scale_inv * b_scale_inv * sum_k val(a[m, k]) * val(b[n, k]) )
 * with fp32 accumulation; the product of the two scale inverses is formed in
 * fp32 and multiplies the accumulators before the epilogue.
 *   a, b             uint8 [M, K] / [N, K] FP8 codes (no block scales)
 *   a_scale_inv, b_scale_inv   float [1] each, device (e.g. q_scale_inv_out
 *                    of te_fp8_cast_delayed_scaling or scale_inv_out of
 *                    te_fp8_cast_current_scaling)
 *   d, d_dtype, bias, aux, shapes: as te_mxfp8_gemm; epi is TE_EPI_NONE,
 *   TE_EPI_BIAS or TE_EPI_BIAS_GELU_AUX; workspace: none is used (NULL / 0).
 */
te_status te_fp8_gemm(const uint8_t* a, const float* a_scale_inv, te_dtype a_fmt,
                      const uint8_t* b, const float* b_scale_inv, te_dtype b_fmt,
                      int64_t M, int64_t N, int64_t K,
                      void* d, te_dtype d_dtype, te_epilogue epi,
                      const uint16_t* bias, uint16_t* aux,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * MXFP8 GEMM with an MXFP8 output: the GEMM and epilogue of te_mxfp8_gemm
 * (NONE, BIAS or BIAS_GELU_AUX), whose D is written as the rowwise MXFP8
 * operand of the next GEMM (the FC1 -> FC2 hand-over of LayerNormMLP: FC1's
 * GELU output is FC2's input) instead of bf16.  The epilogue rounds its fp32
 * results to bf16 exactly as te_mxfp8_gemm with d_dtype TE_BF16 does, then
 * quantizes them in 32-column blocks as te_mxfp8_quantize (TE_ROWWISE) does,
 * so d and d_scale are bit-identical to quantizing that bf16 D.
 *   d        uint8 [M, N] codes, d_fmt TE_E4M3 or TE_E5M2
 *   d_scale  uint8 [M, N/32] E8M0 scales
 *   aux      as te_mxfp8_gemm (bf16 pre-activation, BIAS_GELU_AUX only)
 *   Shapes as te_mxfp8_gemm, and N % 32 == 0; workspace as te_mxfp8_gemm
 *   (te_mxfp8_gemm_workspace_size gives its size).
 */
te_status te_mxfp8_gemm_mxout(const uint8_t* a, const uint8_t* a_scale, te_dtype a_fmt,
                              const uint8_t* b, const uint8_t* b_scale, te_dtype b_fmt,
                              int64_t M, int64_t N, int64_t K,
                              uint8_t* d, uint8_t* d_scale, te_dtype d_fmt, te_epilogue epi,
                              const uint16_t* bias, uint16_t* aux,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Grouped MXFP8 GEMM in one launch ([ROCm-TE] single-launch grouped GEMM /
 * "Grouped GEMM using CK_Tile"; epilogues as te_mxfp8_gemm).  Expert g owns
 * rows [off_g, off_g + m_splits[g]) of A, D and aux, where off_g is the sum
 * of the earlier splits:
 *   D_g = epi(A_g . B_g^T + bias_g).
 *   num_groups  G >= 1
 *   m_splits    int32 [G], DEVICE memory, read by the kernel (no host sync).
 *               Precondition: every split >= 0 and their sum == total_m.
 *               The kernel clamps rows to [0, total_m), so bad splits cannot
 *               write outside D / aux, but their results are unspecified.
 *   a           uint8 [total_m, K], a_scale [total_m, K/32]
 *   b           uint8 [G * N, K] (experts stacked), b_scale [G * N, K/32]
 *   d           [total_m, N] (d_dtype as te_mxfp8_gemm)
 *   bias        bf16 [G, N] iff epi != NONE; aux bf16 [total_m, N] iff GELU-aux
 *   Shapes: total_m >= 0, N % 16 == 0, K % 128 == 0, 0 < K <= 2^23, N > 0.
 *   workspace: none (NULL / 0).
 */
te_status te_mxfp8_grouped_gemm(int32_t num_groups, const int32_t* m_splits, int64_t total_m,
                                const uint8_t* a, const uint8_t* a_scale, te_dtype a_fmt,
                                const uint8_t* b, const uint8_t* b_scale, te_dtype b_fmt,
                                int64_t N, int64_t K,
                                void* d, te_dtype d_dtype, te_epilogue epi,
                                const uint16_t* bias, uint16_t* aux,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Blockwise FP8 quantization ([ROCm-TE] "Blockwise FP8 GEMM support on
 * ROCm": 1-D (1 x 128) blocks for activations and gradients, 2-D
 * (128 x 128) blocks for weights; on gfx950 the recipe's scales are powers
 * of two).  Each block gets scale_inv = the smallest power of two p with
 * amax / p <= the format's largest finite value (448 E4M3, 57344 E5M2), or
 * 1 for an all-zero block; codes are the saturating round-to-nearest-even
 * encodes of x / p (exact division), so no element saturates.
 *   x          bf16 [rows, cols]; cols % 128 == 0, rows >= 0 (any)
 *   fmt        TE_E4M3 or TE_E5M2
 *   block_2d   0: blocks of 128 along each row; scale_inv float [rows, cols/128]
 *              1: 128 x 128 blocks (the last block row may be short);
 *                 scale_inv float [ceil(rows/128), cols/128]
 *   q          uint8 [rows, cols] codes
 *   Inputs holding NaN or Inf give unspecified codes and scales for their
 *   block.  An empty tensor enqueues nothing.
 */
te_status te_fp8_block_quantize(const uint16_t* x, int64_t rows, int64_t cols, te_dtype fmt, int block_2d,
                                uint8_t* q, float* scale_inv, hipStream_t stream);

/*
 * Blockwise FP8 scales cast to MXFP8 scales ([ROCm-TE] "Blockwise FP8 GEMM
 * support on ROCm": on gfx950 the blockwise GEMM computes with the FP32
 * scales cast to E8M0).  A blockwise operand [rows, cols] carries one FP32
 * scale inverse per 1 x 128 block (1-D) or per 128 x 128 block (2-D); its
 * value is code * scale_inv.  Each scale s becomes the E8M0 code of the
 * smallest power of two >= s, saturating at 2^127 (+inf included); +-0 and
 * values up to 2^-127 give 2^-127 (code 0); NaN and negative values give
 * the E8M0 NaN code 255.  Every 32-block inherits its 128-block's code, so
 * the codes with these scales form an MXFP8 operand (exact when every s is
 * a power of two, as the recipe's own scales are).
 *   scale_inv  float [rows, cols/128] (block_2d = 0) or
 *              [ceil(rows/128), cols/128] (block_2d = 1); 4-byte aligned
 *   mx_scale   uint8 [rows, cols/32] E8M0, 4-byte aligned (written)
 *   Shapes: rows >= 0, cols >= 0, cols % 128 == 0; empty enqueues nothing.
 */
te_status te_fp8_block_scales_to_mx(const float* scale_inv, int64_t rows, int64_t cols, int block_2d,
                                    uint8_t* mx_scale, hipStream_t stream);

/*
 * Blockwise FP8 GEMM, "TN" ([ROCm-TE] "Blockwise FP8 GEMM support on ROCm
 * (gfx942 and gfx950)": 1-D x 2-D or 1-D x 1-D block scaling, E4M3 / E5M2
 * inputs except E5M2 x E5M2, bias and DGELU epilogues; an E8M0-cast kernel
 * by default and a kernel taking the FP32 scales):
 *   D[m, n] = epi( sum_kb sa[m, kb] * sb[n, kb] * sum_{k in kb} val(a[m, k]) * val(b[n, k]) )
 * with fp32 accumulation, K blocks kb of 128, and sb read at row n / 128
 * when b_block_2d.
 *   a            uint8 [M, K] codes, a_scale_inv float [M, K/128] (1-D blocks)
 *   b            uint8 [N, K] codes, b_scale_inv float [N, K/128]
 *                (b_block_2d = 0) or [ceil(N/128), K/128] (b_block_2d = 1)
 *   mode         TE_BLOCK_SCALES_E8M0: every scale is cast to E8M0 as
 *                te_fp8_block_scales_to_mx casts it (inside the GEMM kernel):
 *                the result is te_mxfp8_gemm's on the operands with those
 *                scales.
 *                TE_BLOCK_SCALES_FP32: each K block's product is computed
 *                with unit scales and added to the fp32 accumulator times
 *                fl32(sa * sb) with one fused multiply-add; no workspace.
 *   d, d_dtype, epi, bias, aux: as te_mxfp8_gemm (every epilogue), and D
 *                may also be TE_FP16 (IEEE half, round to nearest even; beyond
 *                the half range it becomes +-inf) for every epilogue but
 *                TE_EPI_ACCUMULATE (fp32 D).
 *   beta         TE_EPI_ACCUMULATE: D = fl32(beta * D + acc) with one
 *                rounding (a fused multiply-add; beta = 1 gives D += acc, as
 *                in te_mxfp8_gemm).  Ignored by the other epilogues.
 *   Shapes as te_mxfp8_gemm: K % 128 == 0, M % 16 == 0, N % 16 == 0.
 *   Scale pointers are 4-byte aligned and may be NULL when M, N or K is 0.
 *   workspace    none is needed (te_fp8_block_gemm_workspace_size returns
 *                0); pass NULL / 0.
 */
size_t te_fp8_block_gemm_workspace_size(int64_t M, int64_t N, int64_t K, te_block_scaling mode);
te_status te_fp8_block_gemm(const uint8_t* a, const float* a_scale_inv, te_dtype a_fmt,
                            const uint8_t* b, const float* b_scale_inv, te_dtype b_fmt, int b_block_2d,
                            int64_t M, int64_t N, int64_t K,
                            void* d, te_dtype d_dtype, te_epilogue epi,
                            const uint16_t* bias, uint16_t* aux, te_block_scaling mode, float beta,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TEMX_H */
