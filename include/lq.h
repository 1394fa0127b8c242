/*
 * lq.h -- LoRA / QLoRA adapted linear layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the library liblq.so.  Every entry point takes plain pointers and
 * sizes; device pointers are HIP device memory owned by the caller, contiguous
 * and row-major unless stated.  No call allocates device memory or keeps a
 * pointer after it returns, and none synchronises: work is enqueued on the
 * caller's stream and the call returns.
 *
 * Notation (batched row form): X is M x K, the frozen base W0 is N x K
 * (d_out x d_in), A is r x K, B is N x r, s = alpha / r ("scale"), Y is M x N,
 * T = X A^T (M x r), U = dY B (M x r).
 *
 * Errors: argument problems (null pointer where one is required, a size that
 * is zero where it must not be, an unsupported dtype / shape / rank, a short
 * workspace) are detected before anything is launched and return a negative
 * lq_status; lq_last_error() then gives a message for the calling thread.
 * A failed launch returns LQ_ERR_HIP with HIP's message.  Faults inside a
 * kernel surface at the caller's next synchronisation of the stream.
 *
 * Sources, cited by page title and section:
 *   [MF]  "Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations,
 *          Intrinsic Rank Dynamics, NF4 Quantization, and Parameter-Efficient
 *          Fine-Tuning" (llms.blog)
 *   [FT]  "Large Language Model Fine-tuning and LoRA" (aicomputerinstitute.com)
 *   [UH]  "LoRA and QLoRA fine-tuning under the hood" (codingpancake.com)
 *   [L26] "Lesson 26: LoRA / QLoRA theory" (teology.holyping.network)
 */
#ifndef LQ_H
#define LQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lq_status {
  LQ_OK = 0,
  LQ_ERR_INVALID_ARG = -1,   /* null pointer, bad size, inconsistent metadata   */
  LQ_ERR_UNSUPPORTED = -2,   /* valid request this build does not implement      */
  LQ_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required       */
  LQ_ERR_HIP = -4            /* a HIP call failed; message in lq_last_error()    */
} lq_status;

typedef enum lq_dtype {
  LQ_F32 = 0,                /* IEEE binary32                                    */
  LQ_BF16 = 1                /* bfloat16 (upper half of binary32), RNE stores    */
} lq_dtype;

typedef enum lq_weight_kind {
  LQ_WEIGHT_DENSE = 0,       /* W0 stored densely in ``dtype``                   */
  LQ_WEIGHT_NF4 = 1          /* W0 stored as NF4 codes + block constants         */
} lq_weight_kind;

/* NF4 block sizes fixed by [FT] "Quantizing the frozen weights: NF4 and double
 * quantization" (64 weights per absmax) and [MF] "2. Double Quantization (DQ)"
 * (256 first-level constants per second-level block). */
#define LQ_NF4_BLOCK 64
#define LQ_NF4_DQ_BLOCK 256

/* First-level constant storage (lq_weight.double_quant and the quantiser's
 * double_quant argument):
 *   LQ_DQ_NONE  float32 absmax per block (single-level NF4, 4.5 bits/param;
 *               [FT] "Quantizing the frozen weights")
 *   LQ_DQ_INT8  8-bit integer q = rint(fl32(fl32(c1/c2) * 127)) per block plus
 *               a float32 c2 per 256 blocks ([MF] "2. Double Quantization")
 *   LQ_DQ_FP8   the same bytes holding the E4M3 code nearest (ties to even)
 *               to fl32(fl32(c1/c2) * 127) ([MF] "2. Double Quantization": 8-bit
 *               integers or FP8; [UH] 3.2).  E4M3: 4 exponent bits, bias 7, 3
 *               mantissa bits, subnormals m * 2^-9, max 448.
 * Reconstruction: a' = c1 (NONE), fl32(q * fl32(c2/127)) (INT8),
 * fl32(e4m3(q) * fl32(c2/127)) (FP8). */
#define LQ_DQ_NONE 0
#define LQ_DQ_INT8 1
#define LQ_DQ_FP8 2

/* Codebooks (lq_weight.codebook and the codec's codebook argument):
 *   LQ_CB_NF4            the default: 7 negative levels, an exact 0 and 8
 *                        positive ones (see lq_nf4_codebook)
 *   LQ_CB_NF4_SYMMETRIC  the printed midpoint formula read literally: level
 *                        i = (Q(i/16) + Q((i+1)/16)) / 2 with the infinite end
 *                        quantiles taken at delta and 1 - delta, normalised to
 *                        [-1, 1]; symmetric, no zero ([MF] "1. 4-bit
 *                        NormalFloat (NF4) Quantization"). */
#define LQ_CB_NF4 0
#define LQ_CB_NF4_SYMMETRIC 1

/*
 * The frozen base weight W0, N x K, as seen by every LoRA entry point.
 *
 * kind == LQ_WEIGHT_DENSE: ``dense`` points at N*K elements of ``dtype``.
 * kind == LQ_WEIGHT_NF4: the flattened row-major tensor in NF4 with
 *   codes     ceil(N*K/2) bytes, element 2j in the low nibble of byte j and
 *             element 2j+1 in the high nibble (an odd count leaves the last
 *             high nibble 0);
 *   q8        ceil(N*K/64) bytes (LQ_DQ_INT8: integers 0..127; LQ_DQ_FP8:
 *             E4M3 codes 0..126): 8-bit first-level constants;
 *   c2        ceil(ceil(N*K/64)/256) floats (LQ_DQ_INT8 / LQ_DQ_FP8):
 *             second-level constants;
 *   absmax    ceil(N*K/64) floats (LQ_DQ_NONE): float32 first-level
 *             constants;
 *   the dequantised element is fl32(cb[code] * a') with a' as listed under
 *   LQ_DQ_*, fed to bf16 arithmetic as its round-to-nearest-even bf16 value
 *   ([MF] "1. 4-bit NormalFloat (NF4) Quantization": dequantised to BF16
 *   right before the multiply); cb is the weight's codebook (LQ_CB_*).
 * ``dtype`` for NF4 is the compute dtype the caller intends (checked against
 * the call's dtype).  All pointers are device pointers owned by the caller.
 */
typedef struct lq_weight {
  int32_t kind;              /* lq_weight_kind                                  */
  int32_t dtype;             /* lq_dtype of ``dense`` (dense) / compute (NF4)   */
  int64_t N;                 /* rows, d_out                                     */
  int64_t K;                 /* columns, d_in                                   */
  const void* dense;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* c2;
  const float* absmax;
  int32_t double_quant;      /* LQ_DQ_NONE / LQ_DQ_INT8 / LQ_DQ_FP8             */
  int32_t codebook;          /* LQ_CB_NF4 / LQ_CB_NF4_SYMMETRIC                 */
} lq_weight;

/* --------------------------------------------------------------- NF4 codec */

/*
 * Host copy of the 16 levels of ``codebook`` ([MF] "1. 4-bit NormalFloat
 * (NF4) Quantization": normal quantiles normalised to [-1, 1]), ascending.
 * LQ_CB_NF4 is built on the host in double precision as the asymmetric
 * quantile set with an exact zero (8 positive levels, 7 negative, 0; outer
 * probability 1 - (1/32 + 1/30)/2), LQ_CB_NF4_SYMMETRIC as described above,
 * then rounded to float32.  ``out`` is host memory for 16 floats.
 * Returns LQ_OK or LQ_ERR_INVALID_ARG (null out, unknown codebook).
 */
int lq_nf4_codebook(int32_t codebook, float* out);

/*
 * Quantise n elements of W (flattened, row-major) to NF4
 * ([MF] "1. 4-bit NormalFloat (NF4) Quantization" steps 1-3, and
 * "2. Double Quantization (DQ)"; [FT] "Quantizing the frozen weights").
 *   W        device, n elements of wdt (LQ_F32 or LQ_BF16; bf16 widened
 *            exactly to float32)
 *   blocks of 64 consecutive elements (last may be partial): c1 = max|w|,
 *   x = fl32(w / c1), code = number of the 15 float32 midpoints between
 *   neighbouring levels of ``codebook`` that are strictly below x (c1 = 0:
 *   code 7).
 *   double_quant = LQ_DQ_INT8 or LQ_DQ_FP8: groups of 256 blocks, c2 = max c1
 *   (float32, written to c2[ceil(nb/256)]), y = fl32(fl32(c1/c2) * 127), and
 *   q8 = rint(y) (ties to even) or the E4M3 code nearest y (ties to the even
 *   code); c2 = 0 gives 0; written to q8[nb]; ``absmax`` may be NULL.
 *   double_quant = LQ_DQ_NONE: c1 written to absmax[nb]; q8 and c2 may be NULL.
 *   codes    device, ceil(n/2) bytes (packing as in lq_weight).
 * Results are bit-exact functions of the input.  n >= 1.
 */
int lq_nf4_quantize(const void* W, lq_dtype wdt, int64_t n, int32_t double_quant,
                    int32_t codebook, uint8_t* codes, uint8_t* q8, float* c2, float* absmax,
                    hipStream_t stream);

/*
 * Dequantise n NF4 elements (layout as in lq_weight, format double_quant and
 * codebook as given to lq_nf4_quantize) to ``out``: n elements of odt,
 * fl32(cb[code] * a') for LQ_F32, its RNE bf16 for LQ_BF16.  Bit-exact.  The
 * inverse of lq_nf4_quantize up to the quantisation error.
 */
int lq_nf4_dequantize(const uint8_t* codes, const uint8_t* q8, const float* c2,
                      const float* absmax, int32_t double_quant, int32_t codebook, int64_t n,
                      void* out, lq_dtype odt, hipStream_t stream);

/* ------------------------------------------------------- adapted linear */

/*
 * Forward: Y = X W0^T + s (X A^T) B^T   ([MF] forward-pass equation
 * h = W0 x + (alpha/r) B A x, and the diagram placing alpha/r after B;
 * [UH] 1.2; [L26] "The Decomposition").
 *   X  device M x K of dt;  A device r x K of dt;  B device N x r of dt;
 *   Y  device M x N of dt (written, not accumulated);
 *   T_out  optional device M x r float32: receives T = X A^T for lq_lora_bwd.
 *   ws / ws_bytes: device workspace (caller-owned, contents not preserved).
 *   lq_workspace_size(LQ_OP_FWD, M, N, K, r, 0) bytes select the fastest
 *   path; lq_workspace_size(LQ_OP_FWD_FUSED, ...) is the smallest workspace
 *   that works.  The float32 path needs M r floats of T when T_out is NULL;
 *   otherwise ws may be NULL.
 *   dt = LQ_BF16: bf16 inputs, float32 accumulation, bf16 RNE output; W0 dense
 *   bf16 or NF4.  Paths:
 *     - M <= 16 (decode, memory-bound): one launch, T formed inside it, no
 *       workspace;
 *     - 16 < M <= 64, NF4 W0 with N % 128 == 0 and K % 512 == 0, and at least
 *       the LQ_OP_FWD size: the weight streamed once in (128-row, 512-column)
 *       pieces, float32 partial sums (K/512 M (N + r) floats) in ws, added
 *       in order by a second launch;
 *     - other forwards of up to 96 rows: 16-row chunks, 8 M' r floats of
 *       partial sums of T (M' = M rounded up to a multiple of 16), each chunk
 *       streaming W0 once; with the LQ_OP_FWD workspace and N > 4096 the
 *       chunks stop at 32 rows for an NF4 W0 and at 16 for a bf16 one;
 *     - NF4 W0 with N % 128 == 0, K % 256 == 0 and at least 192 tiles of
 *       128 x 256: one launch that dequantises the codes inside the product's
 *       K loop and forms T there too (no workspace, no dense W0), unless ws
 *       holds the LQ_OP_FWD size and the large-tile product would run
 *       256 x 256 tiles (M > 2816 at N = 4096), where the next case is faster;
 *     - at least the LQ_OP_FWD size, N % 256 == 0: the large-tile path; an
 *       NF4 W0 is first dequantised (bit-exactly, as lq_nf4_dequantize) to a
 *       transient bf16 copy inside ws, then multiplied;
 *     - otherwise the fused kernels (T in the same K loop, NF4 dequantised in
 *       registers / LDS, no dense W0 either).
 *   All give "dequantise, then multiply in bf16" with identical dequantised
 *   values.
 *   Requires K % 64 == 0, N % 64 == 0, N, K <= 65536, M*K and M*N < 2^31,
 *   1 <= r <= 64.
 *   dt = LQ_F32: float32 throughout (W0 dense f32 or NF4), 1 <= r <= 64.
 * M = 0 is a no-op returning LQ_OK.
 */
int lq_lora_fwd(const void* X, int64_t M, const lq_weight* W0, const void* A,
                const void* B, int64_t r, float scale, lq_dtype dt, void* Y,
                float* T_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward ([MF] "Gradient Dynamics and Backpropagation Mechanics", summed
 * over the batch rows; W0 receives no gradient):
 *   dX = dY W0 + s (dY B) A      (optional: dX may be NULL)
 *   dA = s (dY B)^T X            (r x K float32)
 *   dB = s dY^T (X A^T)          (N x r float32)
 *   dA and dB are given together or both NULL; with both NULL only dX is
 *   computed (X and T_saved are then not read).  dX, dA and dB all NULL is
 *   LQ_ERR_INVALID_ARG.
 *   dY device M x N of dt, X device M x K of dt, A and B as in lq_lora_fwd.
 *   T_saved: optional device M x r float32 from lq_lora_fwd's T_out; when
 *   NULL, T is recomputed.
 *   accumulate = 1 adds into dA and dB (gradient accumulation over
 *   micro-batches); 0 overwrites them.
 *   ws / ws_bytes: device workspace of at least
 *   lq_workspace_size(LQ_OP_BWD_FUSED, M, N, K, r, 0) bytes (caller-owned).
 *   dX of an NF4 W0 with K % 256 == 0, N % 128 == 0, r % 8 == 0 and at least
 *   192 tiles of 128 x 256 runs one launch that dequantises the codes inside
 *   its K loop and forms U = dY B there too; with lq_workspace_size(LQ_OP_BWD,
 *   ...) bytes it runs instead, for an NF4 W0 and at most 64 rows, a
 *   weight-streaming kernel, and where the large-tile product would run
 *   256 x 256 tiles (or the weight is dense), the large-tile path (a bf16
 *   copy of an NF4 W0 in ws).
 * Same shape rules as lq_lora_fwd.
 */
int lq_lora_bwd(const void* dY, const void* X, int64_t M, const lq_weight* W0,
                const void* A, const void* B, int64_t r, float scale, lq_dtype dt,
                const float* T_saved, void* dX, float* dA, float* dB,
                int32_t accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * lq_lora_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as lq_lora_bwd with a workspace of exactly
 * LQ_NOALLOC_SCRATCH_BYTES bytes, except that the workspace is a static
 * device array of that size inside the library (one per GPU, held from the
 * library's load until the process ends) rather than a caller buffer.  The
 * call allocates nothing (no hipMalloc / hipFree, no allocating library
 * routine); its first call on a device looks up that device's address of the
 * array once.  A backward whose smallest workspace (the LQ_OP_BWD_FUSED size)
 * exceeds LQ_NOALLOC_SCRATCH_BYTES returns LQ_ERR_WORKSPACE before any
 * launch; where the LQ_OP_BWD size fits as well, dX takes the path that
 * size selects.  All calls on one GPU share the array: calls that overlap in time on
 * one GPU (several streams, several host threads) race and must be ordered
 * by the caller.  Timing (lq_timing_enable) must be off.
 */
#define LQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int lq_lora_bwd_noalloc(const void* dY, const void* X, int64_t M, const lq_weight* W0,
                        const void* A, const void* B, int64_t r, float scale, lq_dtype dt,
                        const float* T_saved, void* dX, float* dA, float* dB,
                        int32_t accumulate, hipStream_t stream);

/*
 * Forward with LoRA-input dropout ([L26] "Putting It Together": the adapter
 * configuration's lora_dropout; the pages give the setting, and the operation
 * is read as inverted dropout on the adapter branch's input):
 *   Y = X W0^T + s (D(X) A^T) B^T,   D(X) = X * keep / (1 - p)
 * The base product sees the undropped X.
 *   keep     device, ceil(M*K/8) bytes: the keep mask drawn by the caller, one
 *            bit per element of X in row-major order, bit j of byte i for
 *            element 8i + j (1 = kept; the caller draws it with probability
 *            1 - p per element)
 *   p        the dropout probability, 0 <= p < 1 (the factor 1/(1 - p) is
 *            formed in double and rounded to float32)
 *   T_out    optional device M x r float32: receives T = D(X) A^T, which
 *            lq_lora_bwd_dropout takes as T_saved
 *   ws       at least lq_workspace_size(LQ_OP_FWD_DROPOUT_FUSED, M, N, K, r, 0)
 *            bytes; lq_workspace_size(LQ_OP_FWD_DROPOUT, ...) bytes select the
 *            large-tile path where it applies (M > 16, N % 256 == 0).
 * Other arguments, shape rules and errors as lq_lora_fwd; dt must be LQ_BF16
 * (LQ_ERR_UNSUPPORTED otherwise).  M = 0 is a no-op.
 */
int lq_lora_fwd_dropout(const void* X, int64_t M, const lq_weight* W0, const void* A,
                        const void* B, int64_t r, float scale, const uint8_t* keep, float p,
                        lq_dtype dt, void* Y, float* T_out, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * Backward of lq_lora_fwd_dropout for the same keep mask and p (the chain
 * rule on its forward; W0 receives no gradient):
 *   dX = dY W0 + s ((dY B) A) * keep / (1 - p)
 *   dA = s (dY B)^T D(X)          (r x K float32)
 *   dB = s dY^T T,  T = D(X) A^T  (N x r float32)
 * T_saved: T_out of the forward with the same mask, or NULL to recompute.
 * ws: at least lq_workspace_size(LQ_OP_BWD_DROPOUT_FUSED, ...) bytes;
 * lq_workspace_size(LQ_OP_BWD_DROPOUT, ...) selects the large-tile dX path.
 * dX / dA / dB / accumulate rules as lq_lora_bwd; dt must be LQ_BF16.
 */
int lq_lora_bwd_dropout(const void* dY, const void* X, int64_t M, const lq_weight* W0,
                        const void* A, const void* B, int64_t r, float scale,
                        const uint8_t* keep, float p, lq_dtype dt, const float* T_saved,
                        void* dX, float* dA, float* dB, int32_t accumulate, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/*
 * DoRA forward ([FT] "Choosing what to adapt": a trained magnitude vector of
 * size d_out times a direction that receives the low-rank update; [MF]
 * "Advanced Variants: DoRA and LoRA+": W = m (V + dW) / ||V + dW||).  The
 * pages disagree on the size of m (d_out vs d_in) and write a Frobenius norm;
 * the reading used is one magnitude per output row and the vector norm of
 * each output row:
 *   W' = diag(m / c) (W0 + s B A),  c_n = ||W0[n] + s B[n] A||_2,
 *   Y = X W'^T = Z * (m / c) per output column,  Z = X (W0 + s B A)^T.
 * W0 enters as the bf16 values the products use (an NF4 base dequantised).
 *   magnitude  device float32[N], m (rows with c_n = 0 are outside the
 *              contract)
 *   Y          device M x N bf16
 *   Z_out      optional device M x N bf16: receives Z, which lq_dora_bwd
 *              needs as Z_saved
 *   T_out      optional device M x r float32: T = X A^T, for lq_dora_bwd
 *   saved_out  optional device float32[lq_dora_saved_floats(N, r)]: receives
 *              the weight-side results c[N], W0 A^T [N x r] and A A^T [r x r],
 *              which lq_dora_bwd can take instead of recomputing them
 *   ws         at least lq_workspace_size(LQ_OP_DORA_FWD_FUSED, M, N, K, r, 0)
 *              bytes; lq_workspace_size(LQ_OP_DORA_FWD, ...) selects the
 *              large-tile product where it applies
 * Shape rules and errors as lq_lora_fwd; dt must be LQ_BF16.  M = 0: no-op.
 */
int lq_dora_fwd(const void* X, int64_t M, const lq_weight* W0, const void* A, const void* B,
                int64_t r, float scale, const float* magnitude, lq_dtype dt, void* Y,
                void* Z_out, float* T_out, float* saved_out, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* Floats of lq_dora_fwd's saved_out buffer: N + N r + r^2. */
int64_t lq_dora_saved_floats(int64_t N, int64_t r);

/*
 * DoRA backward: the exact chain rule through the row norms (the norm is not
 * held constant).  With g = m / c, G' = dY * g (per column) and
 * h_n = sum_m dY[m][n] Z[m][n]:
 *   dm = h / c,  dW = G'^T X + diag(-h m / c^3) (W0 + s B A),
 *   dX = G' (W0 + s B A),  dA = s B^T dW,  dB = s dW A^T.
 *   Z_saved   device M x N bf16, Z_out of lq_dora_fwd on the same inputs
 *   T_saved   optional T_out of that forward (NULL: recomputed)
 *   saved     optional saved_out of that forward, with the same W0, A, B and
 *             scale (NULL: recomputed; the results are the same bits)
 *   dX        optional device M x K bf16
 *   dA, dB, dmag  required float32 outputs (r x K, N x r, N); accumulate = 1
 *             adds into all three
 *   ws        at least lq_workspace_size(LQ_OP_DORA_BWD_FUSED, ...) bytes;
 *             lq_workspace_size(LQ_OP_DORA_BWD, ...) selects the large-tile dX
 * Shape rules and errors as lq_lora_bwd; dt must be LQ_BF16.
 */
int lq_dora_bwd(const void* dY, const void* X, int64_t M, const lq_weight* W0, const void* A,
                const void* B, int64_t r, float scale, const float* magnitude, lq_dtype dt,
                const void* Z_saved, const float* T_saved, const float* saved, void* dX,
                float* dA, float* dB, float* dmag, int32_t accumulate, void* ws,
                size_t ws_bytes, hipStream_t stream);

/*
 * Merge for deployment: W_out = deq(W0) + s B A, N x K of dt
 * ([MF] "1. Static Weight Merging"; [FT] "Merging adapters vs keeping them
 * separate"; [L26] "4. Merging Adapters").  The merged matrix has W0's shape
 * and the compute dtype; float32 accumulation, one rounding to dt.
 */
int lq_lora_merge(const lq_weight* W0, const void* A, const void* B, int64_t r,
                  float scale, lq_dtype dt, void* W_out, hipStream_t stream);

/*
 * Segmented multi-adapter forward on one shared base ([FT] "Serving many
 * adapters at once: the multi-tenant problem"; [MF] "2. Multi-Tenant Dynamic
 * Multiplexing", segmented GEMM):
 *   for each segment i: rows seg_offsets[i] .. seg_offsets[i+1]-1 of X get
 *   Y_i = X_i W0^T + s (X_i A_{id}^T) B_{id}^T with id = seg_adapter[i].
 *   X        device T_tokens x K of dt (bf16)
 *   A_stack  device n_adapters x r x K;  B_stack device n_adapters x N x r
 *   seg_offsets device int32[n_seg+1], seg_adapter device int32[n_seg]
 *   (preconditions: offsets non-decreasing from 0 to T_tokens, ids in
 *   [0, n_adapters); lq_check_segments verifies host copies).
 *   ws: at least lq_workspace_size(LQ_OP_FWD_MULTI_FUSED, T_tokens, N, K, r,
 *   n_adapters) bytes; with lq_workspace_size(LQ_OP_FWD_MULTI, ...) bytes and
 *   N % 256 == 0 the large-tile path runs (adapter-masked
 *   T, then the large product whose expand reads the stacked B).
 *   Requires dt = LQ_BF16, K % 64 == 0, N % 64 == 0, r * n_adapters <= 64.
 */
int lq_lora_fwd_multi(const void* X, int64_t T_tokens, const lq_weight* W0,
                      const void* A_stack, const void* B_stack, int32_t n_adapters,
                      int64_t r, float scale, const int32_t* seg_offsets,
                      const int32_t* seg_adapter, int32_t n_seg, lq_dtype dt,
                      void* Y, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Segmented multi-adapter forward over adapters of different ranks ([FT]
 * "Serving many adapters at once": batched kernels for adapters of different
 * ranks in the same batch, on one possibly quantised base): segment i gets
 *   Y_i = X_i W0^T + scales[a] (X_i A_a^T) B_a^T,  a = seg_adapter[i].
 *   A_cat   device R x K of dt: the adapters' A (r_a x K each) stacked by
 *           rows; adapter a owns rows rank_offsets[a] .. rank_offsets[a+1]-1.
 *   B_cat   device, dt: the adapters' B (N x r_a each, row-major) one after
 *           another; adapter a's starts at element N * rank_offsets[a].
 *   rank_offsets  host int32[n_adapters + 1]: starts at 0, strictly
 *           increasing (every r_a >= 1), R = rank_offsets[n_adapters] <= 64.
 *   scales  host float[n_adapters]: each adapter's alpha_a / r_a.
 *   Segments, W0, dtypes, shape rules and errors as lq_lora_fwd_multi (which
 *   is the case r_a = r, scales[a] = s); ws as
 *   lq_workspace_size(LQ_OP_FWD_MULTI or LQ_OP_FWD_MULTI_FUSED, T_tokens, N,
 *   K, R, 1).  1 <= n_adapters <= 64.
 */
int lq_lora_fwd_multi_ranks(const void* X, int64_t T_tokens, const lq_weight* W0,
                            const void* A_cat, const void* B_cat, int32_t n_adapters,
                            const int32_t* rank_offsets, const float* scales,
                            const int32_t* seg_offsets, const int32_t* seg_adapter,
                            int32_t n_seg, lq_dtype dt, void* Y, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Decode forward of several adapted layers that read the same activations,
 * in one launch: for g < n_layers,
 *   Y[g] = X W[g]^T + s[g] (X A[g]^T) B[g]^T
 * ([MF] 4 "Targeting Attention and MLP Projection Layers": adapters on every
 * linear projection of a block; the query, key and value projections read the
 * same input, and so do the MLP's gate and up projections; [FT] "Which Layers
 * to Adapt").  Each layer's result is that of lq_lora_fwd on the same inputs
 * (up to the summation order of T), with the same decode kernel: every
 * layer's weight is streamed once in one launch, which pays the launch and
 * the first memory round trip once for all of them.
 *   X        device M x K bf16, 0 <= M <= 16 (M = 0 is a no-op)
 *   n_layers 1 .. LQ_DECODE_MAX_LAYERS
 *   W        host array of n_layers weights (device data as in lq_lora_fwd,
 *            bf16 path rules: K % 64 == 0, N % 64 == 0, N, K <= 65536); all
 *            with the same K, kind, constant format and codebook
 *   A, B     host arrays of device pointers: A[g] r x K bf16, B[g] N_g x r
 *   r        1 <= r <= 64, the same for every layer
 *   s        host float[n_layers]: each layer's alpha / r
 *   Y        host array of device pointers: Y[g] M x N_g bf16 (written)
 *   T_out    NULL, or a host array whose entries are NULL or device M x r
 *            float32 (receives T = X A[g]^T)
 * No workspace.  Calls on one stream are ordered; calls that overlap on
 * different streams use different slots of the decode's library memory, as
 * lq_lora_fwd's decode does.  Argument errors return a negative status
 * before any launch.
 */
#define LQ_DECODE_MAX_LAYERS 8
int lq_lora_fwd_decode_layers(const void* X, int64_t M, int32_t n_layers, const lq_weight* W,
                              const void* const* A, const void* const* B, int64_t r,
                              const float* s, void* const* Y, float* const* T_out,
                              hipStream_t stream);

/* ------------------------------------------------- optimizer step (A, B) */

/*
 * One trainable tensor for lq_adamw_step.  All pointers are device memory
 * owned by the caller; master, m, v and weight are updated in place.
 *   master  n float32 master weights
 *   m, v    n float32 first and second moments (zero before step 1)
 *   grad    n gradient elements of the call's gdt (e.g. dA or dB of
 *           lq_lora_bwd, accumulated over micro-batches with accumulate = 1)
 *   weight  optional (NULL: not written): n bf16 working weights, written as
 *           the round-to-nearest-even bf16 of the new master (the A or B the
 *           next lq_lora_fwd reads)
 *   n       element count (0: the entry is skipped and its pointers unused)
 * Vector loads are used when master, m and v are 16-byte aligned, grad is
 * 16-byte (float32) or 8-byte (bf16) aligned and weight 8-byte aligned;
 * other alignments work element by element.
 */
typedef struct lq_adamw_tensor {
  float* master;
  float* m;
  float* v;
  const void* grad;
  void* weight;
  int64_t n;
} lq_adamw_tensor;

/*
 * AdamW step t on the LoRA factors, float32 master weights and moments and a
 * bf16 working copy ([FT] "The real memory ledger": 16 bytes per trainable
 * parameter -- bf16 weight, bf16 gradient, float32 master, m and v; [MF] "The
 * Memory Bottleneck of Full Fine-Tuning").  The pages name AdamW without its
 * formula; the update is decoupled-weight-decay Adam (Loshchilov and Hutter,
 * 2019), element-wise in float32 with g = grad_scale * grad:
 *   p <- p (1 - lr weight_decay)
 *   m <- beta1 m + (1 - beta1) g,   v <- beta2 v + (1 - beta2) g^2
 *   p <- p - (lr / (1 - beta1^t)) m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * The scalar factors are formed in double on the host and rounded once.
 *   tensors   host array of n_tensors descriptors (read during the call only)
 *   gdt       LQ_F32 or LQ_BF16, the gradients' type
 *   step      t >= 1
 *   grad_scale  e.g. 1 / (number of accumulated micro-batches)
 * Requires 0 <= beta1, beta2 < 1, eps >= 0, lr >= 0, weight_decay >= 0, all
 * finite; each n in [0, 2^40]; tensors must not overlap.  n_tensors = 0 is a
 * no-op.  Several tensors go into one launch (up to 24 per launch).
 */
int lq_adamw_step(const lq_adamw_tensor* tensors, int32_t n_tensors, lq_dtype gdt, float lr,
                  float beta1, float beta2, float eps, float weight_decay, int64_t step,
                  float grad_scale, hipStream_t stream);

/* Host-side check of segment metadata (host pointers).  LQ_OK when offsets
 * start at 0, never decrease, end at T_tokens and every id is in range;
 * LQ_ERR_INVALID_ARG otherwise. */
int lq_check_segments(const int32_t* h_offsets, const int32_t* h_adapter,
                      int32_t n_seg, int64_t T_tokens, int32_t n_adapters);

/* Workspace sizes (bytes) for the ops that need one.  LQ_OP_FWD, LQ_OP_BWD
 * and LQ_OP_FWD_MULTI: the size that lets the call take its fastest path
 * (it holds the large-tile path's part, the bf16 copy of W0 and the split-K
 * slots, and the weight-streaming kernels' partial sums, whichever the shape
 * can use); LQ_OP_FWD_FUSED, LQ_OP_BWD_FUSED and
 * LQ_OP_FWD_MULTI_FUSED: the smallest size each call accepts, with which the
 * fused kernels run.  LQ_OP_{FWD,BWD}_DROPOUT and LQ_OP_DORA_{FWD,BWD} and
 * their _FUSED forms: the same pair for the dropout and DoRA entry points
 * (the DoRA sizes assume an NF4 base, whose bf16 copy they include). */
#define LQ_OP_FWD 0
#define LQ_OP_BWD 1
#define LQ_OP_FWD_MULTI 2
#define LQ_OP_FWD_FUSED 3
#define LQ_OP_BWD_FUSED 4
#define LQ_OP_FWD_MULTI_FUSED 5
#define LQ_OP_FWD_DROPOUT 6
#define LQ_OP_FWD_DROPOUT_FUSED 7
#define LQ_OP_BWD_DROPOUT 8
#define LQ_OP_BWD_DROPOUT_FUSED 9
#define LQ_OP_DORA_FWD 10
#define LQ_OP_DORA_FWD_FUSED 11
#define LQ_OP_DORA_BWD 12
#define LQ_OP_DORA_BWD_FUSED 13
size_t lq_workspace_size(int32_t op, int64_t M, int64_t N, int64_t K, int64_t r,
                         int32_t n_adapters);

/* Trainable parameters LoRA adds to one N x K matrix: r (N + K)
 * ([FT] "Choosing what to adapt: targets and rank"). */
int64_t lq_lora_num_params(int64_t N, int64_t K, int64_t r);

/* Message for the last failed call on this thread ("" if none). */
const char* lq_last_error(void);

/*
 * Kernel timing, a measurement aid for benchmarks (not from the pages).  While
 * enabled (on != 0), each launch of the product kernels is bracketed by a
 * pair of HIP events recorded on the launch stream; names: "g256_fwd" and
 * "g256_dx" (large-tile forward and dX products), "fwd_kernel" and
 * "dx_kernel" (fused forward and dX).  Off by default; do not enable it while
 * a stream is being captured into a graph.
 * lq_timing_read waits for the recorded launches of kernel ``name`` and
 * returns the sum of their event-measured durations (milliseconds) and their
 * number, then forgets them.  Host pointers; LQ_ERR_INVALID_ARG on NULL.
 */
int lq_timing_enable(int32_t on);
int lq_timing_read(const char* name, double* total_ms, int64_t* launches);

/*
 * Test aids for the waits in which one workgroup waits for data another
 * workgroup of the same launch publishes: the decode kernel's wait for the
 * partial sums of T, and the split-K partner wait of the large-tile path.
 * Every such wait is bounded, and one that gives up is counted on the device.
 * A decode workgroup that gives up computes T itself from X and A, so the
 * output stays correct.  A split-K workgroup that gives up leaves its
 * partner's partial sums unread, so its output tile holds half of the
 * reduction: a nonzero count means such a call's output is not to be used.
 * Neither happens in normal operation (the partner is already past its own
 * reduction when the wait starts).
 * lq_debug_set_wait_limit: the bound, in polls, for launches made after the
 * call.  polls > 0 sets it; 0 restores the default (2^22 polls, about a tenth
 * of a second); polls < 0 makes every such wait give up at once, which runs
 * the fallbacks deterministically.  Returns LQ_OK.
 * lq_debug_wait_giveups: synchronises the current device, stores in *count
 * the number of waits that gave up on it since the last call, and clears that
 * number.  LQ_ERR_INVALID_ARG if count is NULL; LQ_ERR_HIP on a HIP error.
 */
int lq_debug_set_wait_limit(int32_t polls);
int lq_debug_wait_giveups(int64_t* count);

#ifdef __cplusplus
}
#endif
#endif /* LQ_H */
