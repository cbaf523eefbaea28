/*
 * qmv_oracle.c -- the oracle for the block-quantized matvec path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check of __graft_entry__ and the
 * cpu_baseline leg of bench.py use it.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * Plain, slow, obviously-correct C99 in double precision.  Every function
 * states the definition it writes out.  Sources are the pages collected on
 * the subject:
 *   [NST]  "One Native Stack for Private, Continuously-Learning AI" --
 *          Sec. "The Unified Quant Core" (Q8_0 = symmetric, 34 bytes per 32
 *          weights; Q4_0 = symmetric, 18 bytes per 32 weights; one block
 *          decoder per format dequantizes a stored block to values) and the
 *          QLoRA Lemma of Sec. "The Central Efficiency Thesis"
 *          (y_i = sum_j What_ij x_j with What = DEQ(W)).
 *   [ESP]  "Economical Serving and the hanzo.ai Platform" -- Sec. 2.1 "The
 *          Roofline that Sets the Price" (a decode token streams the weights
 *          once) and Sec. 2.2 (per-format block decoder + traits record).
 *   [ZEN]  "Blue -- porting zen-nano (Qwen3-0.6B) to deterministic on-chain
 *          inference" -- "Quantization recipe": int8 weights and activations,
 *          int32 accumulation, per-output-channel requant by
 *          SaturatingRoundingDoublingHighMul(acc, mult[o]) followed by
 *          RoundingDivideByPOT(., shift[o]) to int8.
 * Where the pages leave a step open (byte layout, nibble order, Q4_1, the
 * Q4_K and Q6_K super-block layouts, the bodies of the two gemmlowp functions, the
 * int8 saturation range) this file takes the plainest reading; each such
 * place says "Reading:".
 *
 * Status: every function below is pinned by the CPU tests (hand-computed
 * blocks and super-blocks, exhaustive fp16 decode, exact-rational brute
 * force, integer closed forms and an independent big-integer mirror).  The
 * Q4_K and Q6_K layouts themselves are readings: agreement with ggml's
 * files is parity unpinned (no ggml file or output is available to compare
 * with).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

enum { QO_Q8_0 = 0, QO_Q4_0 = 1, QO_Q4_1 = 2, QO_Q4_K = 3, QO_Q6_K = 4 };
enum { QO_OK = 0, QO_EINVAL = 1, QO_ENOMEM = 2, QO_EOVERFLOW = 3 };

/* IEEE 754 binary16 -> double, straight from the format definition:
 * bit 15 sign, bits 14..10 biased exponent (bias 15), bits 9..0 fraction.
 * exponent 0: subnormal, value = fraction * 2^-24; exponent 31: inf / NaN;
 * otherwise value = (1024 + fraction) * 2^(exponent - 25).
 * Reading: the pages give "fp16 scales" only; IEEE binary16 is the plain
 * meaning, and subnormals are decoded exactly (no flush). */
double qo_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* Bytes per 32-weight block.  [NST] Sec. "The Unified Quant Core": Q8_0 34
 * bytes, Q4_0 18 bytes.  Q4_1 is not on the pages; reading: fp16 d, fp16 m
 * and 16 bytes of 4-bit codes = 20 bytes. */
int64_t qo_block_bytes(int fmt) {
    switch (fmt) {
    case QO_Q8_0: return 34;
    case QO_Q4_0: return 18;
    case QO_Q4_1: return 20;
    default: return -1;
    }
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Decode one stored block to 32 exact doubles.
 * Reading of the layouts (ggml-compatible, little-endian):
 *   Q8_0: bytes 0-1 d (fp16); bytes 2..33 q_0..q_31 as int8; w_j = d*q_j.
 *   Q4_0: bytes 0-1 d; bytes 2..17 qs[0..15]; element j (j<16) is the low
 *         nibble of qs[j], element j+16 the high nibble; w = d*(c-8).
 *   Q4_1: bytes 0-1 d, bytes 2-3 m (both fp16); bytes 4..19 qs with the
 *         Q4_0 nibble order; w = d*c + m.
 * All three are exact in double: d has at most 11 significant bits, the
 * codes at most 8, and d*c + m spans at most 41 bits. */
void qo_dequant_block(int fmt, const uint8_t* blk, double out[32]) {
    int j;
    if (fmt == QO_Q8_0) {
        double d = qo_f16_to_f64(rd16(blk));
        for (j = 0; j < 32; ++j) out[j] = d * (double)(int8_t)blk[2 + j];
    } else if (fmt == QO_Q4_0) {
        double d = qo_f16_to_f64(rd16(blk));
        for (j = 0; j < 16; ++j) {
            int lo = blk[2 + j] & 0x0f;
            int hi = blk[2 + j] >> 4;
            out[j] = d * (double)(lo - 8);
            out[j + 16] = d * (double)(hi - 8);
        }
    } else {
        double d = qo_f16_to_f64(rd16(blk));
        double m = qo_f16_to_f64(rd16(blk + 2));
        for (j = 0; j < 16; ++j) {
            int lo = blk[4 + j] & 0x0f;
            int hi = blk[4 + j] >> 4;
            out[j] = d * (double)lo + m;
            out[j + 16] = d * (double)hi + m;
        }
    }
}

/* Q4_K: 256-weight super-blocks of 144 bytes.  [NST] Sec. "The Unified
 * Quant Core" lists Q4_K beside Q8_0 and Q4_0 without its layout.
 * Reading: the ggml-compatible layout (agreement with ggml itself is
 * parity unpinned):
 *   bytes 0-1  d    (fp16)   scale of the sub-block scales
 *   bytes 2-3  dmin (fp16)   scale of the sub-block minimums
 *   bytes 4-15 b[0..11]      eight 6-bit scales sc_s and eight 6-bit
 *                            minimums mn_s, s = 0..7:
 *                              s < 4:  sc_s = b[s] & 63,  mn_s = b[s+4] & 63
 *                              s >= 4: sc_s = (b[s+4] & 15) + 16*(b[s-4] >> 6)
 *                                      mn_s = (b[s+4] >> 4) + 16*(b[s] >> 6)
 *   bytes 16-143 q[0..127]   4-bit codes: weight 32s + i (i < 32) is the low
 *                            nibble of q[32*(s/2) + i] for even s, the high
 *                            nibble for odd s
 *   w_{32s+i} = d*sc_s*c - dmin*mn_s.
 * d*sc_s*c (at most 21 significant bits) and dmin*mn_s (at most 17) are
 * exact in double; their difference is exact whenever its bit span is at
 * most 53 (scale exponents within 2^32 of each other), else rounded once. */
static void q4k_scale_min(const uint8_t b[12], int s, int* sc, int* mn) {
    if (s < 4) {
        *sc = b[s] & 63;
        *mn = b[s + 4] & 63;
    } else {
        *sc = (b[s + 4] & 15) + 16 * (b[s - 4] >> 6);
        *mn = (b[s + 4] >> 4) + 16 * (b[s] >> 6);
    }
}

void qo_dequant_superblock_q4k(const uint8_t* sb, double out[256]) {
    double d = qo_f16_to_f64(rd16(sb));
    double dmin = qo_f16_to_f64(rd16(sb + 2));
    const uint8_t* b = sb + 4;
    const uint8_t* q = sb + 16;
    int s, i;
    for (s = 0; s < 8; ++s) {
        int sc, mn;
        q4k_scale_min(b, s, &sc, &mn);
        for (i = 0; i < 32; ++i) {
            int byte = q[32 * (s / 2) + i];
            int c = (s % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
            out[32 * s + i] = d * (double)sc * (double)c - dmin * (double)mn;
        }
    }
}

/* Q6_K: 256-weight super-blocks of 210 bytes, signed 6-bit codes.  [NST]
 * Sec. "The Unified Quant Core" lists it as "signed 6b, 210B/256" without
 * the byte layout.  Reading: the ggml-compatible layout (agreement with
 * ggml itself is parity unpinned):
 *   bytes 0-127    ql[0..127]  low 4 bits of the codes
 *   bytes 128-191  qh[0..63]   high 2 bits of the codes
 *   bytes 192-207  sc[0..15]   int8 scale of each 16-weight sub-block:
 *                              weight e uses sc[e / 16]
 *   bytes 208-209  d (fp16)
 * Weight e = 128 h + 32 q + l (half h < 2, quarter q < 4, l < 32): its low
 * 4 bits are the low nibble (q < 2) or high nibble (q >= 2) of
 * ql[64 h + 32 (q mod 2) + l]; its high 2 bits are bits 2q, 2q+1 of
 * qh[32 h + l]; the 6-bit code c in 0..63 gives
 *   w_e = d * sc[e / 16] * (c - 32).
 * The product has at most 11 + 8 + 6 significant bits: exact in double. */
void qo_dequant_superblock_q6k(const uint8_t* sb, double out[256]) {
    const uint8_t* ql = sb;
    const uint8_t* qh = sb + 128;
    const uint8_t* sc = sb + 192;
    double d = qo_f16_to_f64(rd16(sb + 208));
    int e;
    for (e = 0; e < 256; ++e) {
        int h = e / 128, q = (e % 128) / 32, l = e % 32;
        int lbyte = ql[64 * h + 32 * (q % 2) + l];
        int low4 = (q < 2) ? (lbyte & 0x0f) : (lbyte >> 4);
        int high2 = (qh[32 * h + l] >> (2 * q)) & 3;
        int c = low4 + 16 * high2;
        int scale = (int)(int8_t)sc[e / 16];
        out[e] = d * (double)scale * (double)(c - 32);
    }
}

/* Bytes of one row of K weights; K must be a multiple of the format's
 * block (32, or 256 for the super-block formats). */
int64_t qo_row_bytes(int fmt, int64_t K) {
    if (fmt == QO_Q4_K) return (K % 256) ? -1 : K / 256 * 144;
    if (fmt == QO_Q6_K) return (K % 256) ? -1 : K / 256 * 210;
    if (qo_block_bytes(fmt) < 0 || K % 32) return -1;
    return K / 32 * qo_block_bytes(fmt);
}

/* DEQ(W) for one row of K weights. */
static void dequant_row(int fmt, const uint8_t* row, int64_t K, double* out) {
    int64_t b;
    if (fmt == QO_Q4_K) {
        for (b = 0; b < K / 256; ++b) qo_dequant_superblock_q4k(row + 144 * b, out + 256 * b);
        return;
    }
    if (fmt == QO_Q6_K) {
        for (b = 0; b < K / 256; ++b) qo_dequant_superblock_q6k(row + 210 * b, out + 256 * b);
        return;
    }
    for (b = 0; b < K / 32; ++b) qo_dequant_block(fmt, row + b * qo_block_bytes(fmt), out + 32 * b);
}

/* Full dequantization, row-major [N][K]. */
int qo_dequant(int fmt, const uint8_t* W, int64_t N, int64_t K, double* out) {
    int64_t i, rb = qo_row_bytes(fmt, K);
    if (rb < 0 || N < 0 || K < 0) return QO_EINVAL;
    for (i = 0; i < N; ++i) dequant_row(fmt, W + i * rb, K, out + i * K);
    return QO_OK;
}

/* Float matvec, dequantize-then-dot ([NST] QLoRA Lemma: y_i = sum_j
 * What_ij x_j; [ESP] Sec. 2.1: one pass over the weights per token).
 * For each batch column b and each selected row i:
 *     y[b][t] = sum_{j<K} What_ij * x[b][j]          (sequential j loop)
 *     S[b][t] = sum_{j<K} |What_ij * x[b][j]|
 * where t indexes rows[] (or all rows when rows == NULL).  S is the scale of
 * the acceptance bound |y_gpu - y| <= 1e-4*S + 1e-6.  x rows are ldx floats
 * apart; y and S rows are ldo doubles apart. */
int qo_matvec(int fmt, const uint8_t* W, int64_t N, int64_t K,
              const float* x, int64_t ldx, int32_t B,
              const int64_t* rows, int64_t nrows,
              double* y, double* S, int64_t ldo) {
    int64_t rb = qo_row_bytes(fmt, K), t, j;
    int32_t b;
    double* w;
    if (rb < 0 || N < 0 || K < 0 || B < 0 || ldx < K) return QO_EINVAL;
    if (!rows) nrows = N;
    w = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    if (!w) return QO_ENOMEM;
    for (t = 0; t < nrows; ++t) {
        int64_t i = rows ? rows[t] : t;
        if (i < 0 || i >= N) { free(w); return QO_EINVAL; }
        dequant_row(fmt, W + i * rb, K, w);
        for (b = 0; b < B; ++b) {
            const float* xb = x + (int64_t)b * ldx;
            double acc = 0.0, sabs = 0.0;
            for (j = 0; j < K; ++j) {
                double p = w[j] * (double)xb[j];
                acc += p;
                sabs += fabs(p);
            }
            y[(int64_t)b * ldo + t] = acc;
            if (S) S[(int64_t)b * ldo + t] = sabs;
        }
    }
    free(w);
    return QO_OK;
}

/* floor(n / d) for d > 0, exact in integers. */
static int64_t floor_div(int64_t n, int64_t d) {
    int64_t q = n / d;
    if ((n % d) != 0 && n < 0) q -= 1;
    return q;
}

/* SaturatingRoundingDoublingHighMul(a, b) ([ZEN] "Quantization recipe";
 * the page names the function only, as "int32 multiply-high + rounding
 * shift").  Reading: the high word of the doubled product 2*a*b, i.e.
 * a*b / 2^31, rounded to nearest with ties toward +infinity:
 *     floor((a*b + 2^30) / 2^31),
 * saturating the single overflowing case a = b = -2^31 to 2^31 - 1. */
int32_t qo_srdhm(int32_t a, int32_t b) {
    int64_t p;
    if (a == INT32_MIN && b == INT32_MIN) return INT32_MAX;
    p = (int64_t)a * (int64_t)b;
    return (int32_t)floor_div(p + ((int64_t)1 << 30), (int64_t)1 << 31);
}

/* RoundingDivideByPOT(x, e) ([ZEN] "Quantization recipe", name only).
 * Reading: x / 2^e rounded to nearest, ties away from zero, 0 <= e <= 31. */
int32_t qo_rdbpot(int32_t x, int32_t e) {
    int64_t p, ax, q;
    if (e <= 0) return x;            /* e == 0: identity (callers pass 0..31) */
    p = (int64_t)1 << e;
    ax = x < 0 ? -(int64_t)x : (int64_t)x;
    q = floor_div(2 * ax + p, 2 * p); /* floor(|x|/2^e + 1/2) */
    return (int32_t)(x < 0 ? -q : q);
}

/* Saturate to the int8 range.  Reading: "-> int8" means [-128, 127]. */
int32_t qo_sat8(int32_t v) { return v < -128 ? -128 : (v > 127 ? 127 : v); }

/* The per-output-channel requant of one accumulator ([ZEN]). */
int32_t qo_requant(int32_t acc, int32_t mult, int32_t shift) {
    return qo_sat8(qo_rdbpot(qo_srdhm(acc, mult), shift));
}

/* All-integer matvec with per-output-channel requant ([ZEN]):
 *     acc_i = sum_j Wq_ij * x_j        (exact, int64; must fit int32)
 *     y_i   = sat8(RDBPOT(SRDHM(acc_i, mult_i), shift_i)).
 * acc (optional) receives the int64 accumulators, y the int8 outputs, both
 * indexed [b][t] with row stride ldo.  Returns QO_EOVERFLOW when an
 * accumulator does not fit int32 (the path accumulates in int32). */
int qo_matvec_i8(const int8_t* W, int64_t N, int64_t K,
                 const int8_t* x, int64_t ldx, int32_t B,
                 const int32_t* mult, const int32_t* shift,
                 const int64_t* rows, int64_t nrows,
                 int64_t* acc, int8_t* y, int64_t ldo) {
    int64_t t, j;
    int32_t b;
    int rc = QO_OK;
    if (N < 0 || K < 0 || B < 0 || ldx < K) return QO_EINVAL;
    if (!rows) nrows = N;
    for (t = 0; t < nrows; ++t) {
        int64_t i = rows ? rows[t] : t;
        if (i < 0 || i >= N) return QO_EINVAL;
        if (shift[i] < 0 || shift[i] > 31) return QO_EINVAL;
        for (b = 0; b < B; ++b) {
            const int8_t* xb = x + (int64_t)b * ldx;
            const int8_t* wr = W + i * K;
            int64_t s = 0;
            for (j = 0; j < K; ++j) s += (int64_t)wr[j] * (int64_t)xb[j];
            if (acc) acc[(int64_t)b * ldo + t] = s;
            if (s < INT32_MIN || s > INT32_MAX) { rc = QO_EOVERFLOW; s = 0; }
            y[(int64_t)b * ldo + t] = (int8_t)qo_requant((int32_t)s, mult[i], shift[i]);
        }
    }
    return rc;
}

/* Mixture-of-experts expert matvec, naive form ([NST] Sec. "The Unified
 * Quant Core": each routed expert goes through the same matvec core).
 * For every token b < batch and slot s < top_k, with e = ids[b*top_k + s]:
 *     y[(b*top_k + s)][t] = sum_j DEQ(W_e)_{rows[t], j} * x_{b,s}[j]
 * where W_e starts expert_stride bytes after W_{e-1} and x_{b,s} sits at
 * x + b*x_stride_token + s*x_stride_slot.  No grouping: that is only a
 * schedule.  Ids outside [0, n_experts) are an error here. */
int qo_moe(int fmt, const uint8_t* W, int64_t expert_stride, int32_t n_experts,
           int64_t N, int64_t K, const int32_t* ids, int32_t batch, int32_t top_k,
           const float* x, int64_t x_stride_token, int64_t x_stride_slot,
           const int64_t* rows, int64_t nrows, double* y, double* S, int64_t ldo) {
    int32_t b, s;
    int rc;
    if (!rows) nrows = N;
    for (b = 0; b < batch; ++b) {
        for (s = 0; s < top_k; ++s) {
            int32_t e = ids[b * top_k + s];
            int64_t p = (int64_t)b * top_k + s;
            if (e < 0 || e >= n_experts) return QO_EINVAL;
            rc = qo_matvec(fmt, W + (int64_t)e * expert_stride, N, K,
                           x + b * x_stride_token + s * x_stride_slot, K, 1,
                           rows, nrows, y + p * ldo, S ? S + p * ldo : NULL, ldo);
            if (rc != QO_OK) return rc;
        }
    }
    return QO_OK;
}

/* ------------------------------------------------------------------ the
 * steps on either side of the matvec (fused on the GPU, separate here). */

/* The requantized int8 output mapped through a frozen lookup table.  [ZEN]
 * "Quantization recipe": the integer engine's activation ops run as frozen
 * tables (SiLU among them).  Reading: a table is 256 int8 entries and value
 * v in [-128, 127] maps to lut[v + 128]; the table's contents belong to the
 * caller (a SiLU table folds the activation scales into its entries).
 *     y_i = lut[sat8(RDBPOT(SRDHM(acc_i, mult_i), shift_i)) + 128] */
int qo_matvec_i8_lut(const int8_t* W, int64_t N, int64_t K,
                     const int8_t* x, int64_t ldx, int32_t B,
                     const int32_t* mult, const int32_t* shift, const int8_t* lut,
                     const int64_t* rows, int64_t nrows,
                     int64_t* acc, int8_t* y, int64_t ldo) {
    int64_t t;
    int32_t b;
    int rc = qo_matvec_i8(W, N, K, x, ldx, B, mult, shift, rows, nrows, acc, y, ldo);
    if (rc != QO_OK && rc != QO_EOVERFLOW) return rc;
    if (!rows) nrows = N;
    for (b = 0; b < B; ++b)
        for (t = 0; t < nrows; ++t) {
            int8_t* p = y + (int64_t)b * ldo + t;
            *p = lut[(int)*p + 128];
        }
    return rc;
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).  [ZEN] "Architecture": the MLP
 * is SwiGLU(gate, up, down); the page names it only.  Reading: the standard
 * SwiGLU MLP, h = SiLU(gate x) * (up x), then down h. */
double qo_silu(double z) { return z / (1.0 + exp(-z)); }

/* MoE gate/up with the SwiGLU step ([NST] Sec. "The Unified Quant Core": the
 * MoE path runs each routed expert through the matvec core).  Every expert
 * matrix holds 2F rows: the gate rows 0..F-1, then the up rows F..2F-1 (the
 * caller stores the two row-concatenated).  For pair p = (b, s) with expert
 * e = ids[p] and row i = rows[t]:
 *     g = sum_j DEQ(W_e)_{i, j} x_p[j],   u = sum_j DEQ(W_e)_{F+i, j} x_p[j],
 *     h[p][t] = SiLU(g) * u,
 * with g, u (and their |.| sums Sg, Su) returned as well, all [p][t] with row
 * stride ldo. */
int qo_moe_swiglu(int fmt, const uint8_t* W, int64_t expert_stride, int32_t n_experts,
                  int64_t F, int64_t K, const int32_t* ids, int32_t batch, int32_t top_k,
                  const float* x, int64_t x_stride_token, int64_t x_stride_slot,
                  const int64_t* rows, int64_t nrows,
                  double* h, double* g, double* u, double* Sg, double* Su, int64_t ldo) {
    int32_t b, s;
    int64_t t;
    int rc;
    if (F < 1) return QO_EINVAL;
    if (!rows) nrows = F;
    for (b = 0; b < batch; ++b) {
        for (s = 0; s < top_k; ++s) {
            int32_t e = ids[b * top_k + s];
            int64_t p = (int64_t)b * top_k + s;
            const float* xp = x + b * x_stride_token + s * x_stride_slot;
            if (e < 0 || e >= n_experts) return QO_EINVAL;
            for (t = 0; t < nrows; ++t) {
                int64_t i = rows ? rows[t] : t, ri[2];
                double yv[2], sv[2];
                if (i < 0 || i >= F) return QO_EINVAL;
                ri[0] = i;
                ri[1] = F + i;
                rc = qo_matvec(fmt, W + (int64_t)e * expert_stride, 2 * F, K, xp, K, 1, ri, 1, &yv[0], &sv[0], 1);
                if (rc != QO_OK) return rc;
                rc = qo_matvec(fmt, W + (int64_t)e * expert_stride, 2 * F, K, xp, K, 1, ri + 1, 1, &yv[1], &sv[1], 1);
                if (rc != QO_OK) return rc;
                g[p * ldo + t] = yv[0];
                u[p * ldo + t] = yv[1];
                Sg[p * ldo + t] = sv[0];
                Su[p * ldo + t] = sv[1];
                h[p * ldo + t] = qo_silu(yv[0]) * yv[1];
            }
        }
    }
    return QO_OK;
}

/* MoE down projection with the router-weighted combine of a token's top_k
 * expert outputs (the MoE block's last step).  For token b and row
 * i = rows[t]:
 *     out[b][t] = sum_{s<top_k} w[b][s] * y[b][s][t],
 *     y[b][s][t] = sum_j DEQ(W_{ids[b][s]})_{i, j} x_{b,s}[j],
 *     S[b][t] = sum_s |w[b][s]| * sum_j |DEQ(W_{ids[b][s]})_{i, j} x_{b,s}[j]|.
 * Reading: the router weights are given (the router and its normalization
 * are not part of this step). */
int qo_moe_combine(int fmt, const uint8_t* W, int64_t expert_stride, int32_t n_experts,
                   int64_t N, int64_t K, const int32_t* ids, const float* w, int32_t batch, int32_t top_k,
                   const float* x, int64_t x_stride_token, int64_t x_stride_slot,
                   const int64_t* rows, int64_t nrows, double* out, double* S, int64_t ldo) {
    int32_t b, s;
    int64_t t;
    int rc;
    double *y, *sy;
    if (!rows) nrows = N;
    y = (double*)malloc((size_t)(nrows > 0 ? nrows : 1) * sizeof(double));
    sy = (double*)malloc((size_t)(nrows > 0 ? nrows : 1) * sizeof(double));
    if (!y || !sy) { free(y); free(sy); return QO_ENOMEM; }
    for (b = 0; b < batch; ++b) {
        for (t = 0; t < nrows; ++t) {
            out[(int64_t)b * ldo + t] = 0.0;
            S[(int64_t)b * ldo + t] = 0.0;
        }
        for (s = 0; s < top_k; ++s) {
            int32_t e = ids[b * top_k + s];
            double ws = (double)w[b * top_k + s];
            if (e < 0 || e >= n_experts) { free(y); free(sy); return QO_EINVAL; }
            rc = qo_matvec(fmt, W + (int64_t)e * expert_stride, N, K,
                           x + b * x_stride_token + s * x_stride_slot, K, 1, rows, nrows, y, sy, nrows);
            if (rc != QO_OK) { free(y); free(sy); return rc; }
            for (t = 0; t < nrows; ++t) {
                out[(int64_t)b * ldo + t] += ws * y[t];
                S[(int64_t)b * ldo + t] += fabs(ws) * sy[t];
            }
        }
    }
    free(y);
    free(sy);
    return QO_OK;
}
