/*
 * qmv.h -- block-quantized matrix x vector products for AMD MI355X (gfx950).
 *
 * C ABI of libqmv.so.  Every entry point is asynchronous on the given HIP
 * stream, allocates nothing, keeps no state between calls (apart from a
 * thread-local error message) and is deterministic: the same inputs give
 * bitwise-identical outputs (fixed reduction order, no atomics).
 *
 * Conventions shared by all entry points
 *   - Pointers W, x, y, mult, shift, expert_ids and out are DEVICE pointers
 *     owned by the caller; the library only reads inputs and fully
 *     overwrites outputs.  Outputs must not alias inputs.
 *   - stream is a hipStream_t passed as void*; NULL means the null stream.
 *   - Matrices are row-major.  A block-quantized row of n_cols weights is
 *     n_cols/32 consecutive 32-weight blocks; rows follow each other with no
 *     padding.  Block layouts (ggml-compatible, little-endian):
 *       Q8_0  34 bytes: d (fp16) | q[32] (int8)               w = d*q
 *       Q4_0  18 bytes: d (fp16) | qs[16]                     w = d*(c-8)
 *       Q4_1  20 bytes: d (fp16) | m (fp16) | qs[16]          w = d*c + m
 *     For Q4_0/Q4_1, weight j < 16 of a block is the low nibble of qs[j] and
 *     weight j + 16 the high nibble of qs[j].  Scales are IEEE binary16 and
 *     are decoded exactly (subnormals included).
 *   - The batch width is 1..8: x holds `batch` activation rows, ldx elements
 *     apart; y holds `batch` output rows, ldy elements apart.  Each batch
 *     column is computed independently of the others.  The FMA kernels give
 *     a column bitwise the same result as a batch-1 call on it alone; the
 *     matrix-core kernel (batch 2..8, see qmv_matvec_path) gives a column
 *     bitwise the same result at every batch width 2..8 and position, and
 *     agrees with the batch-1 result within the accuracy contract.  Which
 *     family runs is chosen per shape and batch from measurements (for
 *     the 32-weight formats: the FMA kernels at batch 2 and on rows of up
 *     to 1024 at batch 3..4, the matrix cores from 65536 rows, on longer
 *     matrices at batch 3..4 and from batch 5).
 *   - Float results are fp32, accumulated in fp32; they agree with the exact
 *     dequantize-then-dot within |err| <= 1e-4 * sum_j |w_ij x_j| + 1e-6 per
 *     output (the accuracy contract the tests enforce), for every stored
 *     block and every finite activation vector with 128 * 32 * max|x| below
 *     the fp32 maximum (|x| < 8e34), rows of mostly zero weights included:
 *     no kernel forms a block term as a difference of two sums of size
 *     sum_j |x_j| (Q4_0 dots the signed codes c - 8; Q4_1 dequantizes each
 *     weight, d*c + m, on the FMA kernels, and dots the codes relative to
 *     the block's zero-crossing code on the matrix cores).  The matrix-core
 *     kernel multiplies the codes (exact in bf16) by the activations split
 *     into two bf16 pieces, hi = RN(x) and lo = RN(x - hi), which represent
 *     x to within 2^-16 |x|; the products are exact and summed in fp32.
 *
 * Return codes: QMV_OK on success, otherwise one of QMV_E*, with a message
 * from qmv_last_error().  All argument checks happen on the host before any
 * launch, so a non-OK return means nothing was enqueued (except QMV_EHIP,
 * which reports a failed launch).  Nothing defaults silently.
 *
 * Sources (the pages collected on the subject):
 *   [NST] "One Native Stack for Private, Continuously-Learning AI", Sec. "The
 *         Unified Quant Core": Q8_0 symmetric 34 B/32, Q4_0 symmetric
 *         18 B/32; one templated decode matvec per stage, one block decoder
 *         per format, the same core driving decode and MoE experts; QLoRA
 *         Lemma: y_i = sum_j DEQ(W)_ij x_j accumulated in f32.
 *   [ESP] "Economical Serving and the hanzo.ai Platform", Sec. 2.1 "The
 *         Roofline that Sets the Price" (a decode token streams the resident
 *         weights once; t = W/B) and Sec. 2.2 (quant-agnostic core, block
 *         decoder + traits record, f16/bf16 activation entry points).
 *   [ZEN] "Blue -- porting zen-nano (Qwen3-0.6B) to deterministic on-chain
 *         inference", "Quantization recipe": per-output-channel int8 weights,
 *         int8 activations, int32 accumulation, requant by
 *         SaturatingRoundingDoublingHighMul(acc, mult[o]) then
 *         RoundingDivideByPOT(., shift[o]) to int8.
 *   Q4_1 is not on the pages: its layout above is the ggml-compatible one.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMV_ABI_VERSION 1

typedef enum { QMV_Q8_0 = 0, QMV_Q4_0 = 1, QMV_Q4_1 = 2, QMV_Q4_K = 3, QMV_Q6_K = 4 } qmv_fmt;

enum {
    QMV_OK = 0,
    QMV_EINVAL = 1,       /* null pointer, bad size, batch/top_k out of range */
    QMV_EALIGN = 2,       /* pointer or leading dimension misaligned          */
    QMV_EUNSUPPORTED = 3, /* format not available for this entry point        */
    QMV_EHIP = 4          /* the HIP runtime reported an error at launch      */
};

/*
 * Float block-quantized matvec: y[b][i] = sum_j DEQ(W)[i][j] * x[b][j] for
 * b < batch, i < n_rows ([NST] QLoRA Lemma; [ESP] Sec. 2.1).
 *   W       packed blocks of the format named by the function, n_rows rows of
 *           n_cols/32 blocks; 4-byte aligned.
 *   n_rows  >= 1.
 *   n_cols  >= 32 and a multiple of 32; at most 36384 at batch 1: the FMA
 *           kernels stage one activation row in LDS, 144 bytes per 32
 *           columns, within the 160 KB of a workgroup.  At batch 2..8 longer
 *           rows go to the matrix-core kernel, which stages them in chunks
 *           (n_cols a multiple of 256, and the alignments qmv_matvec_path
 *           lists); otherwise QMV_EINVAL.
 *   x       fp32 [batch][ldx], ldx >= n_cols; 4-byte aligned.
 *   batch   1..8.
 *   y       fp32 [batch][ldy], ldy >= n_rows; 4-byte aligned.
 * Errors: QMV_EINVAL (null pointer, n_rows < 1, n_cols < 32 or not a multiple
 * of 32, batch outside 1..8, ldx < n_cols, ldy < n_rows, n_rows*n_cols/32
 * blocks beyond 2^40, n_cols above the LDS limit on the FMA kernels),
 * QMV_EALIGN (W, x or y not 4-byte aligned), QMV_EHIP.
 */
int32_t qmv_q8_0(const void* W, int64_t n_rows, int64_t n_cols,
                 const float* x, int64_t ldx, int32_t batch,
                 float* y, int64_t ldy, void* stream);
int32_t qmv_q4_0(const void* W, int64_t n_rows, int64_t n_cols,
                 const float* x, int64_t ldx, int32_t batch,
                 float* y, int64_t ldy, void* stream);
int32_t qmv_q4_1(const void* W, int64_t n_rows, int64_t n_cols,
                 const float* x, int64_t ldx, int32_t batch,
                 float* y, int64_t ldy, void* stream);

/*
 * Q4_K float matvec, y[b][i] = sum_j DEQ(W)[i][j] * x[b][j] ([NST] Sec.
 * "The Unified Quant Core" names Q4_K among the core's formats; its layout
 * is not on the pages and is read here as the ggml-compatible one):
 * 256-weight super-blocks of 144 bytes, fp16 d and dmin, eight 6-bit
 * sub-block scales sc_s and minimums mn_s packed in 12 bytes, 128 bytes of
 * 4-bit codes; w_{32s+i} = d*sc_s*c - dmin*mn_s (the byte and bit positions
 * are stated with the kernel, qmv_q4k.hip).
 *   W       n_rows rows of n_cols/256 super-blocks; 16-byte aligned.
 *   n_cols  >= 256 and a multiple of 256; at most 38400 (one activation row
 *           staged in LDS, 68 floats per 64 columns).
 *   x, batch, y as qmv_q8_0.
 * Each weight is dequantized on its own in fp32 (exact scale products, one
 * rounding), so the accuracy bound holds on every input.  Deterministic; on
 * the FMA kernel a column's result is the same bitwise at every batch width.
 * Errors: QMV_EINVAL (as qmv_q8_0, with multiples of 256), QMV_EALIGN (W
 * not 16-byte aligned, x or y not 4-byte aligned), QMV_EHIP.
 * Batch 3..8 may run on the matrix cores (codes about a per-sub-block pivot
 * code, as Q4_1's; within the same bound, columns independent of the batch
 * width among themselves); qmv_matvec_path chooses the family.
 * qmv_matvec_path / qmv_matvec_xt / qmv_dequant accept QMV_Q4_K (matvec on
 * every path; QMV_PATH_MFMA needs batch 2..8, x aligned to 4 elements and
 * ldx a multiple of 4, else QMV_EUNSUPPORTED), and so do the MoE entry
 * points (qmv_moe, qmv_moe_xt, qmv_moe_swiglu, qmv_moe_swiglu_xt,
 * qmv_moe_combine) and qmv_chain / qmv_chain_noalloc.
 */
int32_t qmv_q4_k(const void* W, int64_t n_rows, int64_t n_cols,
                 const float* x, int64_t ldx, int32_t batch,
                 float* y, int64_t ldy, void* stream);

/*
 * Q6_K float matvec, y[b][i] = sum_j DEQ(W)[i][j] * x[b][j] ([NST] Sec.
 * "The Unified Quant Core" lists Q6_K as signed 6-bit, 210 bytes per 256
 * weights; the byte layout is not on the pages and is read here as the
 * ggml-compatible one): 256-weight super-blocks of 210 bytes, 128 bytes of
 * low 4 code bits, 64 of high 2 bits, 16 int8 scales (one per 16 weights),
 * fp16 d; w_e = d*sc[e/16]*(c-32) (bit positions stated with the kernel,
 * qmv_q6k.hip).
 *   W       n_rows rows of n_cols/256 super-blocks; 4-byte aligned.
 *   n_cols  >= 256 and a multiple of 256; at most 38400 (one activation row
 *           staged in LDS, 68 floats per 64 columns).
 *   x, batch, y as qmv_q8_0.
 * Codes are exact signed integers and each 16-weight sum is scaled by the
 * exact d*sc, so the accuracy bound holds on every input.  Deterministic; on
 * the FMA kernel a column's result is the same bitwise at every batch width.
 * Batch 2..8 may run on the matrix cores (sc*(c-32) split exactly into two
 * bf16 pieces; within the same bound, columns independent of the batch
 * width among themselves); qmv_matvec_path chooses the family.
 * Errors: QMV_EINVAL (as qmv_q8_0, with multiples of 256), QMV_EALIGN (W,
 * x or y not 4-byte aligned), QMV_EHIP.
 * qmv_matvec_path / qmv_matvec_xt / qmv_dequant accept QMV_Q6_K (matvec on
 * every path; QMV_PATH_MFMA needs batch 2..8, x aligned to 4 elements and
 * ldx a multiple of 4, else QMV_EUNSUPPORTED), and so do the MoE entry
 * points (qmv_moe, qmv_moe_xt, qmv_moe_swiglu, qmv_moe_swiglu_xt,
 * qmv_moe_combine) and qmv_chain / qmv_chain_noalloc.
 */
int32_t qmv_q6_k(const void* W, int64_t n_rows, int64_t n_cols,
                 const float* x, int64_t ldx, int32_t batch,
                 float* y, int64_t ldy, void* stream);

/*
 * The float matvec above with the kernel family chosen by the caller (a test
 * and tuning aid; the format entry points use QMV_PATH_AUTO):
 *   QMV_PATH_AUTO  the entry point's own choice by shape and batch;
 *   QMV_PATH_FMA   the FMA kernels (one fp32 multiply-add per weight and
 *                  batch column, activations staged in LDS);
 *   QMV_PATH_MFMA  the matrix-core kernel: 16 rows x one 32-weight block x
 *                  up to 8 batch columns per v_mfma_f32_16x16x32_bf16 (the
 *                  block scale applied to its results), for batch 2..8, n_cols
 *                  a multiple of 256, W 16-byte aligned, x 16-byte aligned
 *                  (8-byte for 16-bit activations) and ldx a multiple of 4;
 *                  otherwise QMV_EUNSUPPORTED.
 * Arguments and other errors as the format entry points; QMV_EINVAL for an
 * unknown path, QMV_EUNSUPPORTED for an unknown fmt.
 */
enum { QMV_PATH_AUTO = 0, QMV_PATH_FMA = 1, QMV_PATH_MFMA = 2 };
int32_t qmv_matvec_path(qmv_fmt fmt, const void* W, int64_t n_rows, int64_t n_cols,
                        const float* x, int64_t ldx, int32_t batch,
                        float* y, int64_t ldy, int32_t path, void* stream);

/*
 * The float matvec with 16-bit activations ([ESP] Sec. 2.2: the core is
 * templated on the activation type as well as the weight format, with f16
 * and bf16 entry points).  x holds `batch` rows of x_type elements, ldx
 * elements apart:
 *   QMV_X_F32   fp32 (the same as qmv_matvec_path);
 *   QMV_X_F16   IEEE binary16;
 *   QMV_X_BF16  bfloat16 (the upper half of an fp32).
 * Activations are widened to fp32 exactly and y is fp32, accumulated in fp32:
 * the result equals, bitwise, the fp32 call on the widened activations with
 * the same path.  x must be aligned to its element size; the vectorized
 * staging needs 4-element (8-byte) alignment and ldx a multiple of 4, and is
 * skipped otherwise.  All columns of a call share one pass over W (per
 * column group that fits the LDS, as for fp32).  path as qmv_matvec_path.
 * Errors: as qmv_matvec_path; QMV_EINVAL for an unknown x_type, QMV_EALIGN
 * for x not aligned to its element size.
 */
enum { QMV_X_F32 = 0, QMV_X_F16 = 1, QMV_X_BF16 = 2 };
int32_t qmv_matvec_xt(qmv_fmt fmt, const void* W, int64_t n_rows, int64_t n_cols,
                      const void* x, int32_t x_type, int64_t ldx, int32_t batch,
                      float* y, int64_t ldy, int32_t path, void* stream);

/*
 * All-integer matvec with per-output-channel requant ([ZEN]):
 *   acc[b][i] = sum_j W[i][j] * x[b][j]            (int32, exact)
 *   y[b][i]   = sat_int8(RDBPOT(SRDHM(acc[b][i], mult[i]), shift[i]))
 * SRDHM(a, m) = a*m / 2^31 rounded to nearest, ties toward +infinity, with
 * SRDHM(-2^31, -2^31) = 2^31 - 1; RDBPOT(v, e) = v / 2^e rounded to nearest,
 * ties away from zero; sat_int8 clamps to [-128, 127].
 *   W       int8 [n_rows][n_cols]; 16-byte aligned.
 *   n_cols  >= 16, a multiple of 16, and <= 131056, the largest such value
 *           with n_cols * 128^2 < 2^31, so acc fits int32 for every input.
 *   x       int8 [batch][ldx], ldx >= n_cols and a multiple of 16; 16-byte
 *           aligned.
 *   mult    int32 [n_rows], any value.
 *   shift   int32 [n_rows], each in 0..31 (other values give unspecified
 *           outputs for that row, never an out-of-bounds access).
 *   y       int8 [batch][ldy], ldy >= n_rows.
 * Errors: QMV_EINVAL (null pointer, bad sizes, batch outside 1..8),
 * QMV_EALIGN (W or x not 16-byte aligned, ldx not a multiple of 16), QMV_EHIP.
 */
int32_t qmv_i8_requant(const int8_t* W, int64_t n_rows, int64_t n_cols,
                       const int8_t* x, int64_t ldx, int32_t batch,
                       const int32_t* mult, const int32_t* shift,
                       int8_t* y, int64_t ldy, void* stream);

/*
 * qmv_i8_requant with the requantized outputs mapped through a frozen
 * lookup table, the form in which [ZEN]'s integer engine applies its
 * activation functions (SiLU among them, "Quantization recipe"):
 *   y[b][i] = lut[sat_int8(RDBPOT(SRDHM(acc[b][i], mult[i]), shift[i])) + 128]
 *   lut  int8 [256], device memory, read-only; entry v + 128 is the output
 *        for requantized value v.  Its contents are the caller's (a SiLU
 *        table folds the input and output scales into its entries).
 * Other arguments and errors as qmv_i8_requant; QMV_EINVAL for a null lut.
 */
int32_t qmv_i8_requant_lut(const int8_t* W, int64_t n_rows, int64_t n_cols,
                           const int8_t* x, int64_t ldx, int32_t batch,
                           const int32_t* mult, const int32_t* shift, const int8_t* lut,
                           int8_t* y, int64_t ldy, void* stream);

/*
 * Mixture-of-experts expert matvec ([NST] Sec. "The Unified Quant Core":
 * each routed expert goes through the same decode matvec core).
 * For token b < batch and slot s < top_k, with e = expert_ids[b*top_k + s]:
 *   y[(b*top_k + s)*n_rows + i] = sum_j DEQ(W_e)[i][j] * x_{b,s}[j]
 * where W_e = (const uint8_t*)W_experts + e*expert_stride_bytes is an
 * n_rows x n_cols matrix in format fmt, and
 * x_{b,s} = x + b*x_stride_token + s*x_stride_slot (elements).  Gate/up
 * projections pass x_stride_slot = 0 (one input per token); the down
 * projection passes x_stride_slot = n_cols (one input per token and slot).
 * Each (token, slot) pair is computed as its own matvec (the same sums as a
 * single-expert call, bitwise); an expert routed from several tokens is
 * read from HBM about once and from the GPU's caches for its other pairs.
 * Activations that cannot be staged straight-line (rows of more than 16384
 * columns, or x or its strides not 16-byte aligned) go through a kernel
 * that groups each expert's pairs instead; the results are the same.
 *   fmt                 QMV_Q8_0, QMV_Q4_0, QMV_Q4_1, QMV_Q4_K or QMV_Q6_K.
 *   n_cols              Q8_0 / Q4_0 / Q4_1: a multiple of 32, at most 35488
 *                       (one activation row, 144 bytes per 32 columns, plus
 *                       4 KB of routing tables fit the 160 KB LDS of a
 *                       workgroup).  Q4_K / Q6_K: a multiple of 256, at most
 *                       38400 (1088 bytes of staged row per 256 columns).
 *   expert_stride_bytes >= the bytes of one expert matrix; a multiple of 4
 *                       (of 16 for Q4_K, whose experts are read in 16-byte
 *                       pieces, with W_experts 16-byte aligned).
 *   n_experts           >= 1.
 *   expert_ids          int32 [batch][top_k], device memory.  An id outside
 *                       [0, n_experts) cannot be reported synchronously: the
 *                       n_rows outputs of its (token, slot) are written as
 *                       quiet NaN.
 *   batch               1..8;  top_k 1..16.
 *   x                   fp32; x_stride_token >= n_cols (when batch > 1),
 *                       x_stride_slot 0 or >= n_cols; 4-byte aligned.
 *   y                   fp32 [batch][top_k][n_rows].
 * Errors: QMV_EINVAL, QMV_EALIGN, QMV_EUNSUPPORTED (unknown fmt), QMV_EHIP.
 */
int32_t qmv_moe(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes,
                int32_t n_experts, int64_t n_rows, int64_t n_cols,
                const int32_t* expert_ids, int32_t batch, int32_t top_k,
                const float* x, int64_t x_stride_token, int64_t x_stride_slot,
                float* y, void* stream);

/*
 * qmv_moe with fp32, fp16 or bf16 activations ([ESP] Sec. 2.2: f16 and bf16
 * activation entry points of the one core).  x holds elements of x_type
 * (QMV_X_F32 / QMV_X_F16 / QMV_X_BF16), aligned to the element size; the
 * strides count elements.  Activations are widened to fp32 exactly when
 * staged, so the result equals, bitwise, qmv_moe on the widened values.
 * Errors: as qmv_moe; QMV_EINVAL for an unknown x_type, QMV_EALIGN for x
 * not aligned to its element size.
 */
int32_t qmv_moe_xt(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes,
                   int32_t n_experts, int64_t n_rows, int64_t n_cols,
                   const int32_t* expert_ids, int32_t batch, int32_t top_k,
                   const void* x, int32_t x_type, int64_t x_stride_token, int64_t x_stride_slot,
                   float* y, void* stream);

/*
 * MoE gate/up projection with the SwiGLU step fused ([ZEN] "Architecture":
 * the MLP is SwiGLU(gate, up, down); [NST] Sec. "The Unified Quant Core":
 * each routed expert goes through the same matvec core).  Every expert
 * matrix holds 2*n_ff rows of n_cols: its gate rows 0..n_ff-1, then its up
 * rows n_ff..2*n_ff-1 (the two row-concatenated by the caller).  For token
 * b, slot s, expert e = expert_ids[b*top_k + s] and i < n_ff:
 *   g = sum_j DEQ(W_e)[i][j] * x_{b,s}[j],  u = sum_j DEQ(W_e)[n_ff + i][j] * x_{b,s}[j],
 *   h[(b*top_k + s)*n_ff + i] = SiLU(g) * u,   SiLU(g) = g / (1 + e^-g),
 * with g and u the sums qmv_moe produces for those rows (bitwise), and
 * SiLU and the product in fp32.  Experts are read as in qmv_moe.
 * Arguments as qmv_moe, with expert_stride_bytes >= the bytes of
 * 2*n_ff rows; h is fp32 [batch][top_k][n_ff], 4-byte aligned.  Invalid
 * ids give quiet NaN rows, as in qmv_moe.
 * QMV_Q4_K and QMV_Q6_K experts run it in their super-block kernels (gate
 * row i and up row n_ff + i of a pair in the same lanes and steps).
 * Errors: as qmv_moe.
 */
int32_t qmv_moe_swiglu(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes,
                       int32_t n_experts, int64_t n_ff, int64_t n_cols,
                       const int32_t* expert_ids, int32_t batch, int32_t top_k,
                       const float* x, int64_t x_stride_token, int64_t x_stride_slot,
                       float* h, void* stream);

/* qmv_moe_swiglu with x of x_type, as qmv_moe_xt (h stays fp32). */
int32_t qmv_moe_swiglu_xt(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes,
                          int32_t n_experts, int64_t n_ff, int64_t n_cols,
                          const int32_t* expert_ids, int32_t batch, int32_t top_k,
                          const void* x, int32_t x_type, int64_t x_stride_token, int64_t x_stride_slot,
                          float* h, void* stream);

/*
 * MoE down projection with the router-weighted combine of each token's
 * top_k expert outputs fused (the last step of the MoE block):
 *   out[b*n_rows + i] = sum_{s < top_k} weights[b*top_k + s] * y_{b,s}[i],
 *   y_{b,s}[i] = sum_j DEQ(W_{expert_ids[b*top_k + s]})[i][j] * x_{b,s}[j],
 * with every y_{b,s}[i] the sum qmv_moe produces (bitwise) and the combine
 * an fp32 fused multiply-add chain in slot order s = 0, 1, ...  The router
 * (top-k choice and weight normalization) is the caller's.  Each (token,
 * slot) streams its expert: an expert routed from several tokens is read
 * once per token (no cross-token reduction, so no atomics and no
 * workspace).
 *   weights  fp32 [batch][top_k], device memory, 4-byte aligned.
 *   out      fp32 [batch][n_rows], 4-byte aligned; fully overwritten.
 *   n_cols   144 bytes per 32 columns (one staged slot vector) plus
 *            top_k * 4352 bytes of row sums must fit the 160 KB LDS of a
 *            workgroup (n_cols <= 28608 at top_k = 8).
 * Other arguments as qmv_moe.  A token with an invalid id gets quiet NaN
 * for all its n_rows outputs.
 * QMV_Q4_K and QMV_Q6_K experts run it in a super-block kernel (the
 * batch-1 kernels' row sums; one staged slot vector, 1088 bytes per 256
 * columns, plus top_k * 4100 bytes of row sums within the LDS: n_cols <=
 * 30720 at top_k = 8, 37376 at top_k = 1).
 * Errors: as qmv_moe; QMV_EINVAL for null weights, QMV_EALIGN for
 * misaligned weights.
 */
int32_t qmv_moe_combine(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes,
                        int32_t n_experts, int64_t n_rows, int64_t n_cols,
                        const int32_t* expert_ids, const float* weights, int32_t batch, int32_t top_k,
                        const float* x, int64_t x_stride_token, int64_t x_stride_slot,
                        float* out, void* stream);

/*
 * A chain of batch-1 float matvecs in one call.  Decode is a sequence of
 * matvecs, each streaming its weights once ("Economical Serving and the
 * hanzo.ai Platform", Sec. 2.1); at batch 1 most of them take a few
 * microseconds, about as long as a kernel launch.  Stage s computes
 *   stages[s].y[i] = sum_j DEQ(stages[s].W)[i][j] * stages[s].x[j]
 * for i < n_rows, in format fmt, within the accuracy contract above and
 * deterministically (bitwise the same outputs for the same inputs).  A
 * stage with wait != 0 may read outputs of earlier stages of the same call:
 * it starts reading x only after every earlier stage is complete and its
 * outputs are visible.  A stage with wait == 0 may read only outputs that
 * were already visible to the last earlier stage with wait != 0 (e.g. it
 * shares that stage's input), not outputs of stages after it.  Weight loads
 * of a stage may begin before earlier stages finish.  How it runs:
 *   - at most 4 stages that all read one x with the same n_cols and do not
 *     wait (e.g. the q, k and v projections of a decode step): one matvec
 *     over their concatenated rows, each output bitwise the batch-1 entry
 *     point's for n_cols >= 2048 and a multiple of 2048;
 *   - otherwise, every stage with n_cols a multiple of 2048 and 16-byte
 *     aligned W and x: one persistent launch (per 36 dependency levels)
 *     that streams the weights through LDS and sums each row's 2048-column
 *     window partials in window order (within the bound; not bitwise the
 *     entry points, which accumulate across windows before reducing);
 *   - otherwise one persistent launch of per-stage cursors, each output
 *     bitwise the batch-1 entry point's when n_cols >= 2048.
 *   QMV_Q4_K and QMV_Q6_K stages (n_cols a multiple of 256 up to 38400, W
 *   aligned as for qmv_q4_k / qmv_q6_k) run as launches of their own in
 *   stage order, the stream order standing in for the barriers (the
 *   workspace is checked but not used): each run of up to 4 stages that
 *   read one x with one n_cols and do not wait is one launch over their
 *   concatenated rows; every other stage is the batch-1 entry point's
 *   launch.  Each output is bitwise the batch-1 entry point's.
 *   stages        host array of n_stages entries (copied into the launch).
 *   n_rows        1..2^30;  n_cols a multiple of 32 in 32..35424.
 *   W, x, y       device pointers, 4-byte aligned, as for qmv_q8_0.
 *   workspace     device memory of >= QMV_CHAIN_WORKSPACE_BYTES, 4-byte
 *                 aligned, zero-filled once before its first use; the
 *                 library leaves it ready for the next call.  Calls that
 *                 share a workspace must not run concurrently.  Word 2 is
 *                 an error flag: nonzero means a stage barrier timed out
 *                 (outputs undefined; zero the workspace again).
 * Errors: QMV_EINVAL, QMV_EALIGN, QMV_EUNSUPPORTED (unknown fmt), QMV_EHIP.
 */
#define QMV_CHAIN_WORKSPACE_BYTES 40960
typedef struct {
    const void* W;
    const float* x;
    float* y;
    int64_t n_rows;
    int64_t n_cols;
    int32_t wait;
    int32_t reserved;
} qmv_chain_stage;

int32_t qmv_chain(qmv_fmt fmt, const qmv_chain_stage* stages, int32_t n_stages, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * qmv_chain for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same stages, kernels and outputs as qmv_chain (bitwise), with the chain's
 * barrier words in a library-held device array instead of a caller
 * workspace; the call allocates nothing.
 *   - The array is QMV_CHAIN_WORKSPACE_BYTES (40 KB), a static device
 *     variable of libqmv.so: every GPU the library runs on holds one copy
 *     until the process ends.  Its address is looked up once per device.
 *   - The chain needs the same fixed 40 KB of barrier words for every stage
 *     list, so no list qmv_chain accepts exceeds the array.
 *   - Every call that launches the persistent chain kernel first clears the
 *     array on `stream` with a small kernel (no memset), so a call never
 *     depends on an earlier one, an interrupted one included.
 *   - All calls on one GPU share the array: calls that overlap in time on
 *     one GPU (other streams or threads) race and give undefined outputs;
 *     the caller serializes them.
 * Arguments, outputs and errors as qmv_chain without the workspace, plus
 * QMV_EHIP if the array's address cannot be found.
 */
int32_t qmv_chain_noalloc(qmv_fmt fmt, const qmv_chain_stage* stages, int32_t n_stages, void* stream);

/*
 * Dequantize a whole matrix to fp32: out[i][j] = DEQ(W)[i][j], exactly (every
 * Q8_0/Q4_0 value and every Q4_1 value d*c + m whose bits span <= 24 is
 * representable in fp32; otherwise it is rounded to nearest even; a Q4_K
 * value d*sc*c - dmin*mn is its exact value rounded once; a Q6_K value
 * d*sc*(c-32) is exact).  A test
 * and inspection aid ([NST] Sec. "The Unified Quant Core": the per-format
 * block decoder maps a stored block to its values).
 *   out  fp32 [n_rows][n_cols]; 4-byte aligned.
 * Errors: as the float matvec, plus QMV_EUNSUPPORTED for an unknown fmt.
 */
int32_t qmv_dequant(qmv_fmt fmt, const void* W, int64_t n_rows, int64_t n_cols,
                    float* out, void* stream);

/* Stream-read ceiling (a measurement aid, not a step of the matvec):
 * reads buf[0..bytes) once with 16-byte non-temporal loads, the load form of
 * the whole-line matvec kernel, so that achieved matvec bandwidth can be
 * stated against a read ceiling measured on the same device as well as
 * against the spec ("Economical Serving and the hanzo.ai Platform",
 * Sec. 2.1: spec versus measured achievable read bandwidth; "One Native
 * Stack for Private, Continuously-Learning AI", "Honest Risks": which
 * denominator a figure uses).
 *   buf   device, 16-byte aligned; bytes a positive multiple of 16.
 *   out   device uint32 [out_words], out_words >= 256, 4-byte aligned.
 *         Each of the launch's threads (at most out_words) writes one word,
 *         the XOR of every 32-bit word it read, so the XOR of the written
 *         words equals the XOR of the whole buffer.  Words past the
 *         launch's threads are not written.
 * Errors: QMV_EINVAL (null pointer, bad bytes or out_words), QMV_EALIGN,
 * QMV_EHIP (launch).  Asynchronous on `stream`; the caller owns both buffers.
 */
int32_t qmv_stream_read(const void* buf, size_t bytes, uint32_t* out, size_t out_words, void* stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* qmv_last_error(void);

/* QMV_ABI_VERSION of the built library. */
int32_t qmv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
