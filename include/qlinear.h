/*
 * qlinear.h -- C ABI of the MI355X (gfx950) quantized linear layer.
 *
 * The layer is the fused dequantize-and-multiply of ExLlamaV2's quantized
 * matmul (ExLlamaV2 blog, "How the Fused CUDA Kernel Works"; ExLlamaV2
 * README, "EXL2 quantization"): GPTQ group-wise codes and EXL2 mixed 2/3/4/5/6/8-bit
 * codes, rows remapped by act-order, dequantized as w = s * (q - z) and
 * multiplied against float16 activations with float32 accumulation and a
 * float16 result.
 *
 *   y[m][n] = RNE_fp16( sum_j x[m][perm[j]] * s[g(j)][n] * (q[j][n] - z[g(j)][n]) )
 *
 * Notation: K input features, N outputs, M tokens, gs rows per group
 * (32, 64 or 128), G = K / gs groups, b_g the bit width of group g. Rows of
 * the weight matrix are in *stored order*: stored row j holds the weights of
 * original input feature perm[j] (the act-order permutation).
 *
 * Conventions for every call below:
 *  - All data pointers are DEVICE pointers unless the argument name ends in
 *    _host. Matrices are row-major. The caller allocates and owns every
 *    buffer and every stream; the library allocates nothing, keeps no global
 *    state (but for the static device scratch of qlinear_qgemv_noalloc) and
 *    never synchronizes the host.
 *  - float16 data is passed as uint16_t bit patterns (IEEE binary16).
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously; a QLINEAR_OK return means the launch was accepted.
 *  - Every call validates its host-visible arguments first and returns a
 *    status without launching anything when they are wrong. Device contents
 *    (codes in range, perm being a permutation) are not checked.
 *  - Pointers to device data must be 16-byte aligned (QLINEAR_ERR_MISALIGNED).
 *  - N must be a multiple of 8; K a multiple of gs.
 *  - Non-finite activations: a NaN in row m of x makes row m of y NaN. An
 *    Inf makes every element of its row non-finite. Where the weights are
 *    dequantized exactly the result is the IEEE one of the formula (+-Inf,
 *    NaN where the weight is 0): qlinear_qgemm, and qlinear_qgemv at M >= 3
 *    on layouts where every 32-row block has a scale of its own (groups of
 *    32 or 64 rows, or any width but 4 bits) unless the single-row kernel
 *    takes the call (one width, M = 3 or 4, K N <= 2 * 4096^2, no addend).
 *    The other qlinear_qgemv calls compute the sum in a factored form that
 *    subtracts the activations' block sums (Inf - Inf) and give NaN. Other
 *    rows are unaffected.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call. */
#define QLINEAR_OK 0
#define QLINEAR_ERR_INVALID_ARGUMENT 1 /* NULL pointer, negative or zero size where not allowed */
#define QLINEAR_ERR_UNSUPPORTED 2      /* bit width, group size, M, N or run count outside the supported set */
#define QLINEAR_ERR_MISALIGNED 3       /* a device pointer is not 16-byte aligned */
#define QLINEAR_ERR_WORKSPACE 4        /* workspace missing or smaller than required */
#define QLINEAR_ERR_HIP 5              /* the HIP runtime rejected a launch */

/* Runs of consecutive groups sharing one bit width. Act-order remapping puts
 * the rows quantized at one width next to each other (ExLlamaV2 README,
 * "EXL2 quantization"), so a matrix has only a few runs; up to this many are
 * supported. */
#define QLINEAR_MAX_RUNS 64
/* Largest M accepted by qlinear_qgemv (decode). */
#define QLINEAR_GEMV_MAX_M 16
/* Most matrices in one qlinear_qgemv_grouped call. */
#define QLINEAR_MAX_GROUP 8

/* Activations of the fused epilogue (qlinear_epilogue.activation). */
#define QLINEAR_ACT_NONE 0
#define QLINEAR_ACT_SILU 1 /* v / (1 + exp(-v)), the activation of the Llama MLP */

/*
 * Description of one packed weight matrix: shape, group size and the
 * row-group -> bit-width map, run-length encoded. Filled on the host by
 * qlinear_layout_init and passed by pointer (host memory) to every call.
 *
 * Packed format. Codes are packed into a word matrix of packed_rows x N
 * uint32 words. Each group is cut into 32-row blocks; a block of b-bit codes
 * for one output column is b words, in consecutive packed rows of that
 * column. Group g starts at packed row goff[g] = sum_{g'<g} gs * b_g' / 32,
 * its block c at goff[g] + c * b_g. Inside a block each word is two 16-bit
 * halves (h = 0: bits 0..15, h = 1: bits 16..31) and every code lies inside
 * one half. With f = floor(16 / b) codes per half:
 *   - row r < 2*f*b: word r / (2f); u = r % (2f); half u / f; slot u % f;
 *     code bits at 16*h + b*(u % f) upward. For b = 2, 4, 8 this covers all
 *     32 rows and is the plain least-significant-first order (4-bit: row i of
 *     a word at bits 4i..4i+3, the nibble order of the blog's kernel sketch).
 *   - b = 3, 5: rows 30 + h keep code bit k in word k, bit 16*h + 15.
 *   - b = 6: rows 24 + 4*h + v (v < 4) keep code bits 0..3 in word v at
 *     bits 16*h + 12..15, and code bits 4, 5 in word 4 + v/2 at bits
 *     16*h + 12 + 2*(v % 2) and the bit above it.
 * Storage order: 16-column panels, one after another, each holding its
 * packed rows contiguously: word (r, n) is element ((n/16) * packed_rows + r)
 * * 16 + n % 16 of the uint32 buffer, which holds packed_words =
 * ceil(N/16) * packed_rows * 16 words (panel slots past N are zero).
 */
typedef struct qlinear_layout {
  int32_t K;            /* input features (rows of the weight matrix) */
  int32_t N;            /* output features (columns) */
  int32_t group_size;   /* rows per scale group: 32, 64 or 128 */
  int32_t groups;       /* G = K / group_size */
  int32_t packed_rows;  /* R: rows of the packed word matrix (R x N words) */
  int32_t nruns;        /* number of runs, 1..QLINEAR_MAX_RUNS */
  int32_t run_group[QLINEAR_MAX_RUNS + 1]; /* first group of run r; [nruns] = groups */
  int32_t run_row[QLINEAR_MAX_RUNS + 1];   /* first packed row of run r; [nruns] = packed_rows */
  int32_t run_bits[QLINEAR_MAX_RUNS];      /* code width of run r: 2, 3, 4, 5, 6 or 8 */
  int64_t packed_words;  /* uint32 words of the packed buffer: ceil(N/16) * packed_rows * 16 */
} qlinear_layout;

/* Static, human-readable name of a status code. Never NULL. Every failure is
 * a returned status, where the blog's "Production Considerations" describe
 * the process simply crashing (on out-of-memory). */
const char* qlinear_status_string(int status);

/*
 * Fill `layout` for a K x N matrix with `group_size` rows per group and the
 * per-group bit widths bits_host[0 .. K/group_size - 1]: the q_groups tensor
 * of an EXL2 matrix, a bit width per group (blog, "How the EXL2 Quantization
 * Pipeline Works Under the Hood", Step 3). HOST memory, read
 * only during the call). Host-only; touches no GPU.
 * Errors: INVALID_ARGUMENT (NULL, K <= 0, N <= 0), UNSUPPORTED (group size
 * not 32/64/128, K % group_size != 0, N % 8 != 0, a width outside
 * {2,3,4,5,6,8}, more than QLINEAR_MAX_RUNS runs).
 */
int qlinear_layout_init(qlinear_layout* layout, int32_t K, int32_t N, int32_t group_size,
                        const uint8_t* bits_host);

/*
 * A storage order of the groups under which any per-group width map has at
 * most 6 runs. EXL2 lets each group of a matrix take its own width (blog,
 * "Finding 3: The EXL2 format enables better quality-per-bit") and stores a
 * row permutation with every matrix (blog, "How the EXL2 Quantization
 * Pipeline Works Under the Hood": q_groups and q_invperm). Moving whole
 * groups is a row permutation as well, so a map with more than
 * QLINEAR_MAX_RUNS runs is served by storing its groups in this order.
 * order[i] is the original index of the group stored i-th: widest widths
 * first, original order kept within a width. The caller moves that group's
 * code rows, scale row and zero-point row to position i, and composes the
 * act-order permutation: stored row i * group_size + r takes
 * perm[order[i] * group_size + r], or order[i] * group_size + r without
 * act-order. The product is unchanged up to float rounding order.
 * group_bits (read) and order (written) are HOST arrays of `groups` entries.
 * Host-only; touches no GPU.
 * Errors: INVALID_ARGUMENT (NULL, groups <= 0), UNSUPPORTED (a width outside
 * {2,3,4,5,6,8}); order is not written on error.
 */
int qlinear_group_order(const uint8_t* group_bits, int32_t groups, int32_t* order);

/*
 * Pack codes into the format above: the q_weights tensor, packed values of
 * varying bit width in uint32 words (blog, Step 3 of the EXL2 pipeline), 4-bit
 * codes least significant first as in the blog's kernel sketch ("How the
 * Fused CUDA Kernel Works").
 *   q       : uint8 [K][N], stored row order, each code < 2^b of its group
 *             (larger codes are truncated to their low b bits).
 *   qweight : uint32 [packed_words] in panel order, written entirely.
 */
int qlinear_pack_weights(const qlinear_layout* layout, const uint8_t* q, uint32_t* qweight,
                         void* stream);

/* Inverse of qlinear_pack_weights: qweight -> q uint8 [K][N] (stored order),
 * the unpacking step of the blog's kernel sketch ("How the Fused CUDA Kernel
 * Works") for every width. */
int qlinear_unpack(const qlinear_layout* layout, const uint32_t* qweight, uint8_t* q,
                   void* stream);

/*
 * Dequantize to float16 in stored row order: the group-wise scaling of GPTQ
 * codes (artifact page, GPTQ paragraph: a scale per group) and the sketch's
 * (w - 8) * scale with the zero point generalized (blog, "How the Fused CUDA
 * Kernel Works"):
 *   w[j][n] = RNE_fp16(s[g][n] * (q[j][n] - z[g][n])), g = j / group_size,
 * rounded once (the product is exact before rounding).
 *   scales : float16 [G][N]
 *   zeros  : uint8 [G][N] integer zero points, or NULL for symmetric groups
 *            (z = 2^(b_g - 1), the midpoint of the code range)
 *   w      : float16 [K][N], written entirely.
 */
int qlinear_dequant(const qlinear_layout* layout, const uint32_t* qweight, const uint16_t* scales,
                    const uint8_t* zeros, uint16_t* w, void* stream);

/*
 * Workspace of qlinear_qgemv, in bytes, for any M <= QLINEAR_GEMV_MAX_M: room
 * for the activations gathered into stored row order, the act-order
 * remapping of the README's "EXL2 quantization". For
 * M > 1 it receives the act-order-gathered activations and their 32-row
 * block sums (M = 1 gathers inside the kernel's LDS unless K is very large).
 * It is scratch: no initialization is needed and its contents are not
 * preserved. Calls that may overlap in time (different streams) must not
 * share one workspace.
 */
int qlinear_qgemv_workspace_bytes(const qlinear_layout* layout, size_t* bytes);

/*
 * Decode-sized layer: the fused kernel of the blog's "How the Fused CUDA
 * Kernel Works" (load the quantized weights, dequantize them on the fly and
 * multiply, in one pass with no intermediate weights written), at the token
 * counts of decoding, where the layer is bound by reading its weights (blog,
 * "The Investigation"). 1 <= M <= QLINEAR_GEMV_MAX_M. M == 0 returns OK after
 * checking the layout only, and launches nothing (operands may then be NULL).
 *   x       : float16 [M][K], original feature order
 *   qweight : uint32 [packed_words] from qlinear_pack_weights
 *   scales  : float16 [G][N]
 *   zeros   : uint8 [G][N] or NULL (symmetric)
 *   perm    : int32 [K], stored row j holds feature perm[j]; NULL = identity.
 *             Must be a permutation of 0..K-1 (not checked).
 *   y       : float16 [M][N], written entirely
 *   workspace, workspace_bytes : see qlinear_qgemv_workspace_bytes
 * Errors: as for the layout and pointers above; UNSUPPORTED for M > 16, or
 * for M >= 3 when the scales reach 2^31 bytes (32-bit buffer offsets).
 */
int qlinear_qgemv(const qlinear_layout* layout, const uint16_t* x, int32_t M,
                  const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                  const int32_t* perm, uint16_t* y, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * qlinear_qgemv without a caller-provided workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same operands, result and errors as
 * qlinear_qgemv; the workspace is a static device array of the library (a
 * few MiB, held by each GPU the library runs on until the process ends),
 * found on the calling thread's current device, which `stream` must belong
 * to. Every call on one GPU shares that array: calls that may overlap in
 * time on one GPU (different streams) race and must not be issued. The
 * array needs no clearing between calls. Allocates nothing.
 * Errors: as qlinear_qgemv; UNSUPPORTED also for K > QLINEAR_NOALLOC_MAX_K;
 * HIP if the array's device address cannot be obtained.
 */
#define QLINEAR_NOALLOC_MAX_K 65536
int qlinear_qgemv_noalloc(const qlinear_layout* layout, const uint16_t* x, int32_t M,
                          const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                          const int32_t* perm, uint16_t* y, void* stream);

/*
 * Several decode layers in one launch: count (1 .. QLINEAR_MAX_GROUP) matrices
 * that share the layout, the activations x and the permutation perm -- the
 * projections that read the same input, such as q, k and v, or gate and up
 * (they are quantized against the same input, so act-order gives them the
 * same permutation). One launch amortizes the fixed cost of a kernel over all
 * of them, the point of the blog's fused-QKV kernel ("The Solution",
 * architecture). For each i < count, computes what qlinear_qgemv computes with
 * qweights_host[i], scales_host[i], zeros_host[i] into y_host[i].
 *   qweights_host, scales_host, y_host : HOST arrays of count device pointers
 *   zeros_host : NULL (all symmetric), or a HOST array of count device
 *                pointers, all non-NULL
 * Other arguments and errors as for qlinear_qgemv; INVALID_ARGUMENT also for
 * count < 1 or a zeros array that mixes NULL and non-NULL entries,
 * UNSUPPORTED for count > QLINEAR_MAX_GROUP.
 */
int qlinear_qgemv_grouped(const qlinear_layout* layout, const uint16_t* x, int32_t M, int32_t count,
                          const uint32_t* const* qweights_host, const uint16_t* const* scales_host,
                          const uint8_t* const* zeros_host, const int32_t* perm, uint16_t* const* y_host,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace of qlinear_qgemm for M tokens, in bytes (no initialization needed;
 * the act-order gather of the README's "EXL2 quantization" and the partial
 * sums of layouts with several widths):
 * the gathered activations, float16 [M][K], then float32 partial sums:
 * [M][N] for a layout with several code widths that has at least 16384 rows
 * of K per run boundary when ceil(N / 256) * ceil(M / 256) >= 256 (such a
 * call is computed one launch per run); [S][M][N] when the call cuts K into
 * S = min(16, 1024 / (ceil(N / 128) * ceil(M / 128)), K / 512) > 1 slices
 * (grids of few tiles, activations below 2^31 bytes); the larger of the two.
 * For 17..32 rows at least qlinear_qgemv_workspace_bytes (see qlinear_qgemm). */
int qlinear_qgemm_workspace_bytes(const qlinear_layout* layout, int32_t M, size_t* bytes);

/*
 * Prefill-sized layer, any M >= 0 (M == 0 as for qlinear_qgemv), same
 * operands and result as qlinear_qgemv: the fused kernel on the matrix cores
 * (blog, "How the Fused CUDA Kernel Works": the real kernel uses tensor
 * cores), dequantizing each weight once per tile of tokens.
 * The workspace receives the act-order-gathered activations (and the partial
 * sums described at qlinear_qgemm_workspace_bytes). Calls of 17..32 rows run
 * as two qlinear_qgemv launches (16 rows, then the rest) where the decode
 * kernels support the layout.
 * Errors as for qlinear_qgemv; UNSUPPORTED also for M > 65535 * 128, or for
 * packed words or scales of 2^31 bytes or more.
 */
int qlinear_qgemm(const qlinear_layout* layout, const uint16_t* x, int32_t M,
                  const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                  const int32_t* perm, uint16_t* y, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Output epilogue of the fused calls below: the operations that the GPTQ
 * kernels fuse into the matmul (ExLlamaV2 project page: scaling, addition,
 * activation), applied in float32 to each output before its float16
 * rounding:
 *   y[m][n] = RNE_fp16( act(acc[m][n] + addend[m][n] + bias[n]) + residual[m][n] )
 * where acc is the float32 sum of the plain calls.
 *   bias       : float16 [N], or NULL
 *   residual   : float16 [M][N], or NULL; it may be y itself (in place)
 *   activation : QLINEAR_ACT_NONE or QLINEAR_ACT_SILU
 *   addend     : float32 [M][N], or NULL: a term of the layer's own output,
 *                such as the on-the-fly LoRA update of qlinear_lora_delta
 * HOST struct, read during the call only.
 */
typedef struct qlinear_epilogue {
  const uint16_t* bias;
  const uint16_t* residual;
  int32_t activation;
  const float* addend;
} qlinear_epilogue;

/*
 * qlinear_qgemv and qlinear_qgemm with an output epilogue (NULL = none, the
 * plain call). Same arguments and errors as the plain calls; also
 * UNSUPPORTED for an unknown activation, MISALIGNED for a bias, residual or
 * addend that is not 16-byte aligned.
 */
int qlinear_qgemv_fused(const qlinear_layout* layout, const uint16_t* x, int32_t M,
                        const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                        const int32_t* perm, const qlinear_epilogue* epilogue, uint16_t* y,
                        void* workspace, size_t workspace_bytes, void* stream);
int qlinear_qgemm_fused(const qlinear_layout* layout, const uint16_t* x, int32_t M,
                        const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                        const int32_t* perm, const qlinear_epilogue* epilogue, uint16_t* y,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * EXL2 two-level scales (ExLlamaV2 blog, "How the EXL2 Quantization Pipeline
 * Works Under the Hood", Step 3: q_scale holds 4-bit group scales packed into
 * uint32 words, q_scale_max one float16 maximum scale per output feature;
 * "How the Fused CUDA Kernel Works": a weight dequantizes as
 * (w - midpoint) * scale * scale_max). The pages fix neither the value of a
 * scale code nor the code order; this library reads them as:
 *   scale[g][n] = (c[g][n] + 1) / 16 with c = (q_scale[g][n / 8] >> 4 (n % 8)) & 15
 *   w[j][n]     = (q[j][n] - 2^(b_g - 1)) * scale[g][n] * q_scale_max[n]
 * Groups are symmetric (no zero points).
 *   q_scale     : uint32 [G][N / 8], device
 *   q_scale_max : float16 [N], device
 *
 * qlinear_pack_qscale writes q_scale from 4-bit codes: codes uint8 [groups][N]
 * (device, each taken modulo 16), N a multiple of 8. groups == 0 or N == 0 is
 * a no-op. Errors: INVALID_ARGUMENT for negative sizes or a NULL pointer,
 * UNSUPPORTED for N % 8 != 0, MISALIGNED for pointers not 16-byte aligned.
 *
 * qlinear_dequant_qscale, qlinear_qgemv_qscale and qlinear_qgemm_qscale are
 * qlinear_dequant, qlinear_qgemv_fused and qlinear_qgemm_fused with
 * (q_scale, q_scale_max) in place of (scales, zeros): same layout, operands,
 * workspace, epilogue (NULL = none) and errors, and also INVALID_ARGUMENT
 * for a NULL q_scale or q_scale_max, MISALIGNED for either not 16-byte
 * aligned. The dequantized float16 weight is the single rounding of the
 * exact product. The matmuls weigh each group by c + 1 and multiply the
 * float32 sum by q_scale_max[n] / 16 before the epilogue.
 */
int qlinear_pack_qscale(const uint8_t* codes, int32_t groups, int32_t N, uint32_t* q_scale, void* stream);
int qlinear_dequant_qscale(const qlinear_layout* layout, const uint32_t* qweight, const uint32_t* q_scale,
                           const uint16_t* q_scale_max, uint16_t* w, void* stream);
int qlinear_qgemv_qscale(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                         const uint32_t* q_scale, const uint16_t* q_scale_max, const int32_t* perm,
                         const qlinear_epilogue* epilogue, uint16_t* y, void* workspace, size_t workspace_bytes,
                         void* stream);
int qlinear_qgemm_qscale(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                         const uint32_t* q_scale, const uint16_t* q_scale_max, const int32_t* perm,
                         const qlinear_epilogue* epilogue, uint16_t* y, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Q4 / Q6 / Q8 KV-cache codec (ExLlamaV2 blog: Q4, Q6 and Q8 cache modes next
 * to FP16, "How to Use Effectively", Step 2, where Q8 saves 50% of the cache
 * memory and Q4 75%). The pages give no format; this library's is:
 *   x      : float16 [rows][D], rows of D values (e.g. one head's key or
 *            value vector per token), cut into blocks of `group` elements
 *   scales : float16 [rows][D / group], s = RNE_fp16(max|x| / (2^(bits-1) - 1))
 *            of each block, computed in float32
 *   codes  : uint32 [rows][D * bits / 32]: per block a little-endian bit
 *            stream, element i at bits bits*i .. bits*i + bits - 1, holding
 *            clamp(rint(x / s), -2^(bits-1), 2^(bits-1) - 1) + 2^(bits-1)
 *            (float32 division, ties to even; a block with s = 0 holds the
 *            midpoint code)
 *   dequantized value: RNE_fp16(s * (code - 2^(bits-1)))
 * bits in {4, 6, 8}; group in {32, 64, 128}; D a multiple of group. Stored
 * bytes per element: bits / 8 + 2 / group (Q4 at group 128: 25.8% of FP16).
 * Inputs must be finite. A cache of several heads, layers or tokens is one
 * call with rows = their product; appending one token is a call on that
 * token's rows (pointers offset by the caller).
 * Pointers are device pointers: x 16-byte aligned, codes 4-byte aligned,
 * scales 2-byte aligned (else MISALIGNED). rows == 0 is a no-op.
 * Errors: INVALID_ARGUMENT for rows < 0, D < 1 or a NULL pointer (rows > 0);
 * UNSUPPORTED for other bits or group, D % group != 0, or rows * D above 2^42.
 * Asynchronous on `stream`.
 */
int qlinear_kv_quant(const uint16_t* x, int64_t rows, int32_t D, int32_t bits, int32_t group, uint32_t* codes,
                     uint16_t* scales, void* stream);
int qlinear_kv_dequant(const uint32_t* codes, const uint16_t* scales, int64_t rows, int32_t D, int32_t bits,
                       int32_t group, uint16_t* x, void* stream);

/*
 * On-the-fly LoRA update of a linear layer (ExLlamaV2 project page, LoRA
 * adapters: the low-rank pair A, B is applied during the forward pass
 * instead of being merged into the weights, and several adapters combine
 * with weights):
 *   delta[m][n] = scale * sum_j (sum_k x[m][k] * A[k][j]) * B[j][n]      (accumulate == 0)
 *   delta[m][n] += that                                                  (accumulate != 0)
 * computed with float32 products and sums (x A first, then times B). Pass
 * delta as qlinear_epilogue.addend so that the update joins the layer's sum
 * before bias, activation and the one float16 rounding; call again with
 * accumulate != 0 for each further adapter.
 *   x      : float16 [M][K], the layer's input in its original feature order
 *            (the adapter multiplies x itself, not the act-order gather)
 *   lora_a : float16 [K][rank];  lora_b : float16 [rank][N]
 *   rank   : 1 .. QLINEAR_LORA_MAX_RANK
 *   delta  : float32 [M][N], written (or added to)
 *   workspace : device scratch of qlinear_lora_workspace_bytes(M, K, rank)
 *            bytes (partial sums of x A); contents not preserved
 * M == 0 is a no-op. Errors: INVALID_ARGUMENT for M < 0, K < 1, N < 1, rank
 * < 1 or a NULL pointer (M > 0); UNSUPPORTED for rank above
 * QLINEAR_LORA_MAX_RANK or K or N above QLINEAR_LORA_MAX_DIM; MISALIGNED as
 * for the other calls; WORKSPACE for a workspace that is missing or too
 * small.
 */
#define QLINEAR_LORA_MAX_RANK 64
#define QLINEAR_LORA_MAX_DIM (65535 * 256) /* largest K and N */
int qlinear_lora_workspace_bytes(int32_t M, int32_t K, int32_t rank, size_t* bytes);
int qlinear_lora_delta(const uint16_t* x, int32_t M, int32_t K, const uint16_t* lora_a, int32_t rank,
                       const uint16_t* lora_b, int32_t N, float scale, int32_t accumulate, float* delta,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement helper (not part of the layer): the streaming-read floor that
 * frames the decode kernels' bandwidth, since decode is bound by reading the
 * weights (ExLlamaV2 blog, "The Investigation": the GPU mostly waits on
 * memory). Reads `bytes` of device memory at `buf` once, with
 * `loads_per_thread` (4, 8 or 16) 16-byte loads in flight per thread, over
 * `workgroups` workgroups of 256 threads striding through the buffer, and
 * folds the words into one value per thread, which is written to sink[0]
 * only if it equals `key` (pick a key the data does not produce: nothing is
 * then written). Asynchronous on `stream`.
 * Errors: INVALID_ARGUMENT (NULL, bytes < 16 or not a multiple of 16),
 * UNSUPPORTED (loads_per_thread, workgroups outside 1..65535), MISALIGNED.
 */
int qlinear_read_floor(const void* buf, size_t bytes, int32_t loads_per_thread, int32_t workgroups, uint32_t key,
                       uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
