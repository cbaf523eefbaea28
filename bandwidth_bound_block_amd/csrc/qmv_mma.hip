// Batch 2..8 block-quantized matvec on the matrix cores (gfx950).
//
// The block dot of the quantized-matvec pages (dequantize in registers, dot
// in f32, per-block scale) turns compute-bound once several activation
// columns share each weight: the FMA kernels spend B multiply-adds per
// weight.  Here one v_mfma_f32_16x16x32_bf16 computes, for one 32-weight
// block column, the code dots of 16 rows against 16 activation columns, and
// the per-block scale is applied to its four results per lane afterwards.
//
// Exactness of the operands:
//  * codes (Q8_0 int8, Q4_x nibbles 0..15) have at most 8 significant bits:
//    exact in bf16;
//  * each activation x is split into two bf16 pieces, hi = RN(x) and
//    lo = RN(x - hi) (x - hi is exact in f32), so |x - hi - lo| <= 2^-16 |x|;
//  * bf16 products are exact in f32 and the matrix core sums in f32.
// So each row's result differs from the exact dequantize-then-dot value by at
// most 2^-16 of sum_j |w_j x_j| plus f32 summation error.
//
// MFMA roles: A (16 x 32) = activation pieces, row bp = p*B + b for piece p
// of batch column b (rows past 2B are ignored); B (32 x 16) = codes of 16 weight
// rows.  Lane l supplies A row l%16 and B column l%16 for k-group l/16, and
// holds D[4*(l/16)+i][l%16], i = 0..3: weight row l%16, so the lane scales
// its four results by the fp16 scale of the block of its own row.  Which
// element of the block sits in which k-slot is free as long as A and B agree;
// Mma<F> fixes it per format (x0/x1 below).
//
// Work split: 16-row tiles; a workgroup of NW waves handles NW/KP tiles at a
// time (a tile group) and the KP waves of a tile take interleaved steps of 8
// blocks along the row; their partial sums are combined through LDS in a
// fixed order.  The activation pieces of up to KC blocks are staged in LDS
// (re-staged per tile group when the row needs several chunks).  Each wave
// streams a step (16 rows x 8 blocks) as whole 16-byte chunks into its LDS
// slot, with the next step's loads in flight in registers.
#include <type_traits>

#include "qmv_block_decode.h"

namespace qmv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Calls fn(std::integral_constant<int, J>{}) for J = 0..N-1 in order.
template <class Fn, int... Js>
__device__ __forceinline__ void static_for(std::integer_sequence<int, Js...>, Fn&& fn) {
    (fn(std::integral_constant<int, Js>{}), ...);
}

// Keeps the compiler from folding a nibble mask into per-element bit-field
// extracts (one v_cvt_f32_ubyte<k> per element instead of two instructions).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
// bf16 pair {a, b} (a in the low half) from two floats that are exact in bf16.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_amdgcn_perm(fbits(b), fbits(a), 0x07060302u);
}
__device__ __forceinline__ uint32_t lds4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// Per-format B operand: lane group g (0..3) of weight row r gets 8 codes of
// block J of the row's step (the step's bytes at `row`, in LDS, 16-byte
// aligned), as packed bf16, plus the block's scale (and minimum).
// x0(g), x1(g): the block elements of those 8 codes, as two runs of 4.
template <class F> struct Mma;

template <> struct Mma<Q8_0> {
    static constexpr bool kSums = false;     // the term needs no activation sums
    static constexpr float kOutScale = 1.f;
    __device__ static constexpr int x0(int g) { return 8 * g; }
    __device__ static constexpr int x1(int g) { return 8 * g + 4; }
    // codes q[8g..8g+7] = bytes 2+8g..9+8g of the block; 34j = 2j (mod 4)
    template <int J>
    __device__ static void operand(const uint8_t* row, int g, uint32_t (&b)[4], float& d, float&) {
        const uint8_t* blk = row + 34 * J;
        uint32_t c0, c1;
        if constexpr ((J & 1) == 0) {
            const uint8_t* p = blk + 8 * g;     // 4-aligned; codes start 2 bytes in
            const uint32_t w0 = lds4(p), w1 = lds4(p + 4), w2 = lds4(p + 8);
            c0 = __builtin_amdgcn_alignbyte(w1, w0, 2);
            c1 = __builtin_amdgcn_alignbyte(w2, w1, 2);
        } else {
            const uint8_t* p = blk + 2 + 8 * g;  // 4-aligned
            c0 = lds4(p);
            c1 = lds4(p + 4);
        }
        d = half_bits_to_float(*reinterpret_cast<const uint16_t*>(blk));
        b[0] = pack_bf16(sbyte(c0, 0), sbyte(c0, 1));
        b[1] = pack_bf16(sbyte(c0, 2), sbyte(c0, 3));
        b[2] = pack_bf16(sbyte(c1, 0), sbyte(c1, 1));
        b[3] = pack_bf16(sbyte(c1, 2), sbyte(c1, 3));
    }
    __device__ static float term(float acc, float d, float, float dot, float) { return __builtin_fmaf(d, dot, acc); }
};

template <> struct Mma<Q4_0> {
    static constexpr bool kSums = false;
    static constexpr float kOutScale = 0.0625f;   // the operand carries the codes times 16
    __device__ static constexpr int x0(int g) { return 4 * g; }
    __device__ static constexpr int x1(int g) { return 16 + 4 * g; }
    // qs[4g..4g+3] = bytes 2+4g..5+4g of the block: elements 4g..4g+3 (low
    // nibbles) and 16+4g..19+4g (high nibbles); 18j = 2j (mod 4).  A nibble c
    // placed in the top half of a byte with its top bit flipped reads as the
    // signed byte 16 (c - 8), so one sign-extending convert per code gives
    // the offset code times 16 (exact in bf16; the 16 is taken out once per
    // output, exactly).
    template <int J>
    __device__ static void operand(const uint8_t* row, int g, uint32_t (&b)[4], float& d, float&) {
        const uint8_t* blk = row + 18 * J;
        uint32_t c;
        if constexpr ((J & 1) == 0) {
            const uint8_t* p = blk + 4 * g;
            c = __builtin_amdgcn_alignbyte(lds4(p + 4), lds4(p), 2);
        } else {
            c = lds4(blk + 2 + 4 * g);
        }
        d = half_bits_to_float(*reinterpret_cast<const uint16_t*>(blk));
        const uint32_t lo = ((c << 4) & 0xf0f0f0f0u) ^ 0x80808080u, hi = (c & 0xf0f0f0f0u) ^ 0x80808080u;
        b[0] = pack_bf16(sbyte(lo, 0), sbyte(lo, 1));
        b[1] = pack_bf16(sbyte(lo, 2), sbyte(lo, 3));
        b[2] = pack_bf16(sbyte(hi, 0), sbyte(hi, 1));
        b[3] = pack_bf16(sbyte(hi, 2), sbyte(hi, 3));
    }
    // d * 16 * sum_e (c_e - 8) x_e
    __device__ static float term(float acc, float d, float, float dot, float) { return __builtin_fmaf(d, dot, acc); }
};

// Q4_1 weights d c + m are not exact in bf16, so the operand carries codes
// relative to a pivot code k of the block, the code nearest the zero of
// d c + m (k = clamp(rint(-m/d), 0, 15)):
//   sum_e (d c_e + m) x_e = d sum_e (c_e - k) x_e + mu sum_e x_e,  mu = m + d k.
// c - k is exact in bf16, and both terms stay bounded by the block's
// sum_e |w_e x_e|: where c_e != k, |mu| <= |d|/2 (unless k was clamped, when
// every weight has the sign of mu and |mu| <= |w_e|) and so
// |d (c_e - k)| <= 2 |w_e|; where c_e = k, w_e = mu.  So a block of mostly
// zero weights (d c + m = 0) adds no large cancelling terms.  Any k in
// 0..15 gives the same exact value; the reciprocal only picks it.
template <> struct Mma<Q4_1> {
    static constexpr bool kSums = true;      // mu multiplies the block sum of x
    static constexpr float kOutScale = 1.f;
    __device__ static constexpr int x0(int g) { return 4 * g; }
    __device__ static constexpr int x1(int g) { return 16 + 4 * g; }
    // d: the block's scale; m: returns mu = m + d k
    template <int J>
    __device__ static void operand(const uint8_t* row, int g, uint32_t (&b)[4], float& d, float& m) {
        const uint8_t* blk = row + 20 * J;   // always 4-aligned
        const uint32_t dm = lds4(blk);
        d = half_bits_to_float(dm);
        const float mn = half_bits_to_float(dm >> 16);
        // fmax/fmin return the number for a NaN operand (d = m = 0): k = 0
        const float k = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(-mn * __builtin_amdgcn_rcpf(d)), 0.f), 15.f);
        m = __builtin_fmaf(d, k, mn);
        const uint32_t c = lds4(blk + 4 + 4 * g);
        const uint32_t lo = opaque(c & 0x0f0f0f0fu), hi = opaque((c >> 4) & 0x0f0f0f0fu);
        b[0] = pack_bf16(ubyte(lo, 0) - k, ubyte(lo, 1) - k);
        b[1] = pack_bf16(ubyte(lo, 2) - k, ubyte(lo, 3) - k);
        b[2] = pack_bf16(ubyte(hi, 0) - k, ubyte(hi, 1) - k);
        b[3] = pack_bf16(ubyte(hi, 2) - k, ubyte(hi, 3) - k);
    }
    // d * sum_e (c_e - k) x_e + mu * sum_e x_e
    __device__ static float term(float acc, float d, float mu, float dot, float sx) {
        return __builtin_fmaf(mu, sx, __builtin_fmaf(d, dot, acc));
    }
};

// Q4_K super-blocks (144 bytes per 256 weights: 18 bytes per 32-weight
// sub-block on average, so a step of 8 blocks is one super-block and the row
// pitch is nb * 18).  The 16-byte header holds d, dmin and the 6-bit
// scale and minimum of each sub-block J; its weights are D c - M with
// D = d sc_J and M = dmin mn_J (both exact in fp32), codes in the low (J
// even) or high (J odd) nibbles of bytes 16 + 32 (J / 2) .. +32.  As for
// Q4_1, the operand carries c - k about the code k nearest the zero of
// D c - M (k = clamp(rint(M / D), 0, 15)), and mu = D k - M (rounded once,
// |mu| <= |w_e| wherever c_e != k, and mu = w_e where c_e = k) multiplies
// the block sum of x.  Rows of mostly zero weights (M = D k) give mu = 0.
struct Q4KSuper {
    static constexpr int kBytes = 18;       // per 32 weights, on average
};
template <> struct Mma<Q4KSuper> {
    static constexpr bool kSums = true;
    static constexpr float kOutScale = 1.f;
    __device__ static constexpr int x0(int g) { return 8 * g; }
    __device__ static constexpr int x1(int g) { return 8 * g + 4; }
    template <int J>
    __device__ static void operand(const uint8_t* row, int g, uint32_t (&b)[4], float& d, float& m) {
        const uint32_t h0 = lds4(row), h1 = lds4(row + 4), h2 = lds4(row + 8), h3 = lds4(row + 12);
        // b[i] is byte i % 4 of h1 (i < 4), h2 (i < 8), h3
        constexpr int t = 8 * (J & 3);
        int sc, mn;
        if constexpr (J < 4) {
            sc = (int)((h1 >> t) & 63);
            mn = (int)((h2 >> t) & 63);
        } else {
            sc = (int)(((h3 >> t) & 15) | (((h1 >> (t + 6)) & 3) << 4));
            mn = (int)(((h3 >> (t + 4)) & 15) | (((h2 >> (t + 6)) & 3) << 4));
        }
        const float D = half_bits_to_float(h0) * (float)sc;
        const float M = half_bits_to_float(h0 >> 16) * (float)mn;
        // fmax/fmin return the number for a NaN operand (D = M = 0): k = 0
        const float k = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(M * __builtin_amdgcn_rcpf(D)), 0.f), 15.f);
        d = D;
        m = __builtin_fmaf(D, k, -M);
        const uint8_t* q = row + 16 + 32 * (J >> 1) + 8 * g;
        const uint32_t w0 = lds4(q), w1 = lds4(q + 4);
        const uint32_t c0 = opaque((J & 1) ? ((w0 >> 4) & 0x0f0f0f0fu) : (w0 & 0x0f0f0f0fu));
        const uint32_t c1 = opaque((J & 1) ? ((w1 >> 4) & 0x0f0f0f0fu) : (w1 & 0x0f0f0f0fu));
        b[0] = pack_bf16(ubyte(c0, 0) - k, ubyte(c0, 1) - k);
        b[1] = pack_bf16(ubyte(c0, 2) - k, ubyte(c0, 3) - k);
        b[2] = pack_bf16(ubyte(c1, 0) - k, ubyte(c1, 1) - k);
        b[3] = pack_bf16(ubyte(c1, 2) - k, ubyte(c1, 3) - k);
    }
    // D * sum_e (c_e - k) x_e + mu * sum_e x_e
    __device__ static float term(float acc, float d, float mu, float dot, float sx) {
        return __builtin_fmaf(mu, sx, __builtin_fmaf(d, dot, acc));
    }
};

// A wave step: 16 rows x SB blocks, read as whole 16-byte chunks.
template <class F, int SB>
struct MmaStep {
    static constexpr int kRowStep = SB * F::kBytes;
    static constexpr int kChunksPerRow = kRowStep / 16;
    static constexpr int kChunks = 16 * kChunksPerRow;
    static constexpr int kLoads = (kChunks + 63) / 64;
    static constexpr int kSlot = 16 * kRowStep;                 // LDS bytes per wave
    static_assert(kRowStep % 16 == 0, "whole chunks per row step");
    static_assert(kSlot >= 16 * 20 * 4, "the slot also holds a wave's 16 x 16 partial sums (rows of 20)");
    struct Buf {
        u32x4 v[kLoads];
    };
};

// Splits x into bf16 pieces for blocks [b0, b0 + nbc) of every batch column
// and stores them in the A-operand layout: row q = g*2B + bp (k-group g,
// piece row bp) holds the 16-byte operand of each block of the chunk, kcp
// entries apart (kcp odd: the 16 lanes of a k-group hit distinct banks).
// For Q4_1 also the block sums of each piece row, as rows g of four floats
// (piece rows 4g..4g+3).  One thread per (column, block) with blocks
// fastest: it does all four k-groups (the sums need no cross-lane step), and
// neighbouring lanes write neighbouring 16-byte entries of a row.
template <class F, int NT, class XT>
__device__ __forceinline__ void stage_pieces(const XT* __restrict__ x, int64_t ldx, int B, int b0, int nbc,
                                             int kcp, uint8_t* xs, float* sxs) {
    using M = Mma<F>;
    for (int idx = threadIdx.x; idx < nbc * B; idx += NT) {
        const int b = idx / nbc, blk = idx - b * nbc;
        const XT* src = x + b * ldx + 32 * (b0 + blk);
        float sums[2][4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 u = XIn<XT>::load4(src + M::x0(g));
            const float4 w = XIn<XT>::load4(src + M::x1(g));
            const float v[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
            uint32_t hp[4], lp[4];
            float sh = 0.f, sl = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // one packed convert per pair: hi = RN(x), then lo = RN(x - hi)
                const float a = v[2 * k], c = v[2 * k + 1];
                hp[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, c}, bf16x2));
                const float ha = __builtin_bit_cast(float, hp[k] << 16);
                const float hc = __builtin_bit_cast(float, hp[k] & 0xffff0000u);
                lp[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a - ha, c - hc}, bf16x2));
                if constexpr (M::kSums) {
                    sh += ha;
                    sh += hc;
                    sl += __builtin_bit_cast(float, lp[k] << 16);
                    sl += __builtin_bit_cast(float, lp[k] & 0xffff0000u);
                }
            }
            const int qh = g * 2 * B + b;   // hi piece row b, lo piece row B + b
            *reinterpret_cast<u32x4*>(xs + (qh * kcp + blk) * 16) = u32x4{hp[0], hp[1], hp[2], hp[3]};
            *reinterpret_cast<u32x4*>(xs + ((qh + B) * kcp + blk) * 16) = u32x4{lp[0], lp[1], lp[2], lp[3]};
            sums[0][g] = sh;
            sums[1][g] = sl;
        }
        if constexpr (M::kSums) {
            const float sh = (sums[0][0] + sums[0][1]) + (sums[0][2] + sums[0][3]);
            const float sl = (sums[1][0] + sums[1][1]) + (sums[1][2] + sums[1][3]);
            sxs[((b >> 2) * kcp + blk) * 4 + (b & 3)] = sh;
            sxs[(((B + b) >> 2) * kcp + blk) * 4 + ((B + b) & 3)] = sl;
        }
    }
}

template <class F, int NW, int SB, int PD, class XT = float>
__global__ __launch_bounds__(64 * NW) void qmv_mma_kernel(const uint8_t* __restrict__ W, int N, int nb,
                                                          const XT* __restrict__ x, int64_t ldx, int B,
                                                          float* __restrict__ y, int64_t ldy, int KP, int KC) {
    using M = Mma<F>;
    using S = MmaStep<F, SB>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int TPI = NW / KP, ts = wave / KP, kp = wave % KP;
    const int nsteps = nb / SB;
    const int tiles = (N + 15) >> 4;
    const int ngroups = (tiles + TPI - 1) / TPI;
    const int CS = KC / SB;                             // steps per chunk (a multiple of KP)
    const int nchunks = (nsteps + CS - 1) / CS;
    const int ipg = nsteps / KP;                        // items (steps) per wave per tile group
    const int ipc = CS / KP;                            // items per wave per full chunk
    const int kcp = KC | 1;                             // entries per piece row (odd)
    const int64_t pitch = (int64_t)nb * F::kBytes;

    uint8_t* xs = lds;                                            // [4 * 2B][kcp] x 16 B
    float* sxs = reinterpret_cast<float*>(xs + 128 * B * kcp);    // [ceil(2B/4)][kcp] x 4 floats (Q4_1)
    uint8_t* slots = reinterpret_cast<uint8_t*>(sxs) + (M::kSums ? 16 * ((2 * B + 3) / 4) * kcp : 0);
    uint8_t* slot = slots + wave * S::kSlot;

    // A operand: piece row bp = lane % 16, k-group lane / 16.  Lanes past the
    // 2B piece rows read a valid row too; their results are never used.
    const int g = lane >> 4, r = lane & 15;
    const uint8_t* a_base = xs + (g * 2 * B + r % (2 * B)) * kcp * 16;
    // block sums for the lane's result rows bp = 4g..4g+3 (rows past 2B unused)
    const uint8_t* s_base = reinterpret_cast<const uint8_t*>(sxs) + (4 * g < 2 * B ? g : 0) * kcp * 16;

    // Chunk k of a step: row k / kChunksPerRow, 16-byte column k % kChunksPerRow.
    int roff[S::kLoads], coff[S::kLoads];
#pragma unroll
    for (int k = 0; k < S::kLoads; ++k) {
        const int i = min(64 * k + lane, S::kChunks - 1);
        roff[k] = i / S::kChunksPerRow;
        coff[k] = 16 * (i % S::kChunksPerRow);
    }
    const int my_groups = (ngroups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int total = my_groups > 0 ? my_groups * ipg : 0;

    // Loads step n (past the last one: the last one again, so that every
    // pipeline slot issues its loads unconditionally and the waits before
    // each LDS copy count exactly the loads issued after it).  pitch < 2^24.
    auto load = [&](int n, typename S::Buf& buf) __attribute__((always_inline)) {
        n = min(n, total - 1);
        const int it = blockIdx.x + (n / ipg) * gridDim.x;
        const int s = kp + KP * (n % ipg);
        // wave-uniform base row (clamped) and 32-bit lane offsets from it:
        // rows past the end re-read the last row
        const int brow = min(16 * (it * TPI + ts), N - 1);
        const int lim = N - 1 - brow;
        const uint8_t* base = W + (int64_t)brow * pitch + (int64_t)s * S::kRowStep;
#pragma unroll
        for (int k = 0; k < S::kLoads; ++k) {
            const uint32_t o = __umul24((uint32_t)min(roff[k], lim), (uint32_t)pitch) + (uint32_t)coff[k];
            buf.v[k] = *reinterpret_cast<const u32x4*>(base + o);
        }
    };
    auto to_slot = [&](const typename S::Buf& buf) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < S::kLoads; ++k)
            if (64 * k + 64 <= S::kChunks || 64 * k + lane < S::kChunks)
                *reinterpret_cast<u32x4*>(slot + 16 * (64 * k + lane)) = buf.v[k];
    };

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    struct Dot {
        f32x4 dot, sx;
        float d, m;
    };
    // Operands of block J of the step and its MFMA; the scaling follows one
    // block later, so the matrix core's latency is covered.
    auto issue = [&](auto jc, int cb) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        Dot o;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(a_base + cb * 16);
        o.sx = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (M::kSums) o.sx = *reinterpret_cast<const f32x4*>(s_base + cb * 16);
        uint32_t bw[4];
        o.m = 0.f;
        M::template operand<J>(slot + r * S::kRowStep, g, bw, o.d, o.m);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        o.dot = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bw), z, 0, 0, 0);
        return o;
    };
    auto finish = [&](const Dot& o) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = M::term(acc[i], o.d, o.m, o.dot[i], o.sx[i]);
    };

    auto item = [&](int n) __attribute__((always_inline)) {
        const int nig = n % ipg;
        const int c = nig / ipc;
        if (nig % ipc == 0 && (nchunks > 1 || n == 0)) {
            const int b0 = c * KC;
            __syncthreads();
            stage_pieces<F, 64 * NW, XT>(x, ldx, B, b0, min(KC, nb - b0), kcp, xs, sxs);
            __syncthreads();
        }
        const int cb = (kp + KP * nig) * SB - c * KC;   // first block of the step in the chunk
        Dot dots[SB];
        static_for(std::make_integer_sequence<int, SB>{}, [&](auto jc) __attribute__((always_inline)) {
            constexpr int J = decltype(jc)::value;
            dots[J] = issue(jc, cb + J);
            if constexpr (J > 0) finish(dots[J - 1]);
        });
        finish(dots[SB - 1]);
        if (nig == ipg - 1) {
            // tile group done: partials of every wave through the slots
            const int it = blockIdx.x + (n / ipg) * gridDim.x;
            __syncthreads();
            // rows of 20 floats: the 16-byte stores and the reads below hit distinct banks
            *reinterpret_cast<f32x4*>(slot + (r * 20 + 4 * g) * 4) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            __syncthreads();
            const int outs = TPI * 16 * B;
            for (int t = tid; t < outs; t += 64 * NW) {
                const int tsl = t / (16 * B), rem = t % (16 * B), b = rem >> 4, rr = rem & 15;
                const int row = 16 * (it * TPI + tsl) + rr;
                float v = 0.f;
                for (int q = 0; q < KP; ++q) {
                    const float* pw = reinterpret_cast<const float*>(slots + (tsl * KP + q) * S::kSlot) + rr * 20;
                    v += pw[b];
                    v += pw[B + b];
                }
                if (row < N) y[b * ldy + row] = v * M::kOutScale;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = 0.f;
        }
    };

    // PD register buffers: the loads of the next PD - 1 steps are in flight
    // while a step is computed.
    if (total == 0) return;
    typename S::Buf buf[PD];
    static_for(std::make_integer_sequence<int, PD - 1>{}, [&](auto pc) __attribute__((always_inline)) {
        load(decltype(pc)::value, buf[decltype(pc)::value]);
    });
    for (int n = 0; n < total; n += PD) {
        bool done = false;
        static_for(std::make_integer_sequence<int, PD>{}, [&](auto pc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value;
            if (done || n + P >= total) {
                done = true;
                return;
            }
            load(n + P + PD - 1, buf[(P + PD - 1) % PD]);
            __builtin_amdgcn_sched_barrier(0);
            to_slot(buf[P]);
            item(n + P);
        });
    }
}

template <class F, int NW, int SB, int PD, class XT = float>
bool launch_mma(const uint8_t* W, int64_t N, int nb, const XT* x, int64_t ldx, int B, float* y, int64_t ldy,
                hipStream_t st, int kp_force, int32_t* rc) {
    using S = MmaStep<F, SB>;
    if (nb % SB) return false;
    const int nsteps = nb / SB;
    const size_t fixed = (size_t)NW * S::kSlot;
    // LDS per staged block (plus one block of padding per chunk)
    const size_t per_blk = 128 * (size_t)B + (Mma<F>::kSums ? 16 * (size_t)((2 * B + 3) / 4) : 0);
    if (fixed + (SB + 1) * per_blk > (size_t)kLdsMax) return false;
    const int64_t tiles = (N + 15) / 16;
    const int cus = device_cu_count();
    int KP = 1;
    if (kp_force > 0) {
        KP = kp_force;
        if (NW % KP || nsteps % KP) return false;
    } else {
        while (KP < NW && nsteps % (2 * KP) == 0 && (tiles + NW / KP - 1) / (NW / KP) < cus) KP *= 2;
    }
    // steps per chunk: a multiple of KP (fewer waves per tile if KP steps do not fit)
    int cs_max = 0;
    for (;; KP /= 2) {
        cs_max = (int)((kLdsMax - fixed) / per_blk - 1) / SB / KP * KP;
        if (cs_max >= KP) break;
        if (KP == 1) return false;
    }
    const int nchunks = (nsteps + cs_max - 1) / cs_max;
    const int cs = ((nsteps + nchunks - 1) / nchunks + KP - 1) / KP * KP;
    const int KC = cs * SB;
    const size_t lds = fixed + (size_t)(KC | 1) * per_blk;

    auto kern = qmv_mma_kernel<F, NW, SB, PD, XT>;
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv", &dyn_max)) {
        *rc = e;
        return true;
    }
    if (lds > dyn_max) {
        *rc = fail(QMV_EINVAL, "qmv: %zu bytes of staged activations exceed the LDS", lds);
        return true;
    }
    const int64_t ngroups = (tiles + NW / KP - 1) / (NW / KP);
    const int per_cu = resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds);
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ngroups, (int64_t)cus * per_cu));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, W, (int)N, nb, x, ldx, B, y, ldy, KP, KC);
    *rc = check_launch("qmv");
    return true;
}

// Q6_K on the matrix cores.  Its weights are d sc (c - 32) with an int8
// scale per 16 weights, so a 32-wide MFMA step spans two scales: the scale
// goes into the B operand.  p = 4 (c - 32) sc is an integer of at most 15
// bits (exact in fp32) and splits exactly into two bf16 pieces, hi =
// RN_bf16(p) and lo = p - hi (at most 7 significant bits); both pieces are
// multiplied into one accumulator per super-block, and d / 4 (exact) scales
// its sum.  No operand is rounded, so the bound is that of the split
// activations, as for the other formats.  The weights go straight to
// registers: 210-byte super-blocks start 2 bytes past a word at every other
// index, so each 8-byte piece is read as 4-byte-aligned words (16 bytes
// from 0 or 2 bytes before it, inside the super-block or the one before)
// and re-aligned with v_alignbyte.  A wave step is one super-block of 16
// rows: lane (g, r) takes row r and, of each 32-weight chunk j = 4 h + q,
// the codes 8g..8g+7 (low 4 bits from ql[64 h + 32 (q & 1) + 8 g ..], high
// 2 bits from qh[32 h + 8 g ..]).
struct Q6KSuper {};
template <> struct Mma<Q6KSuper> {
    static constexpr bool kSums = false;
    __device__ static constexpr int x0(int g) { return 8 * g; }
    __device__ static constexpr int x1(int g) { return 8 * g + 4; }
};

struct Q6KLane {
    u32x4 ql[4];        // [2 h + (q & 1)]: ql bytes 64 h + 32 (q & 1) + 8 g - sh .. +16
    u32x4 qh[2];        // [h]: qh bytes 32 h + 8 g - sh .. +16
    u32x4 t;            // bytes 192 - sh .. +16 (the scales)
    uint32_t u, dh, sh; // sc[14..15], d, 0 or 2
};

__device__ __forceinline__ void q6k_lane_fetch(const uint8_t* sb, int g, Q6KLane& r) {
    const int sh = (int)(reinterpret_cast<uintptr_t>(sb) & 2);
    const uint8_t* p = sb - sh;
#pragma unroll
    for (int k = 0; k < 4; ++k) r.ql[k] = ld16(p + 64 * (k >> 1) + 32 * (k & 1) + 8 * g);
#pragma unroll
    for (int h = 0; h < 2; ++h) r.qh[h] = ld16(p + 128 + 32 * h + 8 * g);
    r.t = ld16(p + 192);
    r.u = ld2(sb + 206);
    r.dh = ld2(sb + 208);
    r.sh = (uint32_t)sh;
}

// 4 (c - 32) for four codes of quarter q as signed bytes: lo holds their 4
// low bits at bits 0-3 (q < 2) or 4-7, hf the qh word with the top bit of
// every 2-bit field flipped.
__device__ __forceinline__ uint32_t q6k_code_bytes(uint32_t lo, uint32_t hf, int q) {
    const uint32_t l = q < 2 ? (lo << 2) : (lo >> 2);
    const uint32_t h = (hf << (6 - 2 * q)) & 0xc0c0c0c0u;
    return (l & 0x3c3c3c3cu) | h;
}

template <int NW, class XT>
__global__ __launch_bounds__(64 * NW) void q6k_mma_kernel(const uint8_t* __restrict__ W, int N, int nsb,
                                                          const XT* __restrict__ x, int64_t ldx, int B,
                                                          float* __restrict__ y, int64_t ldy, int KP, int KC) {
    constexpr int kSlot = 16 * 20 * 4;                  // a wave's 16 x 16 partial sums (rows of 20)
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int TPI = NW / KP, ts = wave / KP, kp = wave % KP;
    const int nb = 8 * nsb;                             // 32-weight blocks per row
    const int tiles = (N + 15) >> 4;
    const int ngroups = (tiles + TPI - 1) / TPI;
    const int CS = KC / 8;                              // super-blocks per chunk (a multiple of KP)
    const int nchunks = (nsb + CS - 1) / CS;
    const int ipg = nsb / KP;                           // items per wave per tile group
    const int ipc = CS / KP;                            // items per wave per full chunk
    const int kcp = KC | 1;
    const int64_t pitch = (int64_t)nsb * 210;

    uint8_t* xs = lds;                                  // [4 * 2B][kcp] x 16 B
    uint8_t* slots = xs + 128 * B * kcp;
    uint8_t* slot = slots + wave * kSlot;

    const int g = lane >> 4, r = lane & 15;
    const uint8_t* a_base = xs + (g * 2 * B + r % (2 * B)) * kcp * 16;
    const int my_groups = (ngroups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int total = my_groups > 0 ? my_groups * ipg : 0;

    // Loads item n (past the last one: the last one again, so every pipeline
    // slot loads unconditionally); rows past the end re-read the last row.
    auto load = [&](int n, Q6KLane& buf) __attribute__((always_inline)) {
        n = min(n, total - 1);
        const int it = blockIdx.x + (n / ipg) * gridDim.x;
        const int s = kp + KP * (n % ipg);
        const int row = min(16 * (it * TPI + ts) + r, N - 1);
        q6k_lane_fetch(W + (int64_t)row * pitch + (int64_t)s * 210, g, buf);
    };

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    auto item = [&](int n, const Q6KLane& w) __attribute__((always_inline)) {
        const int nig = n % ipg;
        const int c = nig / ipc;
        if (nig % ipc == 0 && (nchunks > 1 || n == 0)) {
            const int b0 = c * KC;
            __syncthreads();
            stage_pieces<Q6KSuper, 64 * NW, XT>(x, ldx, B, b0, min(KC, nb - b0), kcp, xs, nullptr);
            __syncthreads();
        }
        const int cb = (kp + KP * nig) * 8 - c * KC;   // first block of the super-block in the chunk
        uint32_t L[4][2], H[2][2], S[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            L[k][0] = __builtin_amdgcn_alignbyte(w.ql[k].y, w.ql[k].x, w.sh);
            L[k][1] = __builtin_amdgcn_alignbyte(w.ql[k].z, w.ql[k].y, w.sh);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            H[h][0] = __builtin_amdgcn_alignbyte(w.qh[h].y, w.qh[h].x, w.sh) ^ 0xaaaaaaaau;
            H[h][1] = __builtin_amdgcn_alignbyte(w.qh[h].z, w.qh[h].y, w.sh) ^ 0xaaaaaaaau;
        }
        {
            const uint32_t t5[5] = {w.t.x, w.t.y, w.t.z, w.t.w, w.u};
#pragma unroll
            for (int i = 0; i < 4; ++i) S[i] = __builtin_amdgcn_alignbyte(t5[i + 1], t5[i], w.sh);
        }
        const int sb_sh = 8 * (g >> 1);
        f32x4 dsum = {0.f, 0.f, 0.f, 0.f};
        static_for(std::make_integer_sequence<int, 8>{}, [&](auto jc) __attribute__((always_inline)) {
            constexpr int J = decltype(jc)::value, h = J >> 2, q = J & 3;
            // scale sc[2 J + g / 2]
            const float sc = (float)(int8_t)(S[J >> 1] >> (16 * (J & 1) + sb_sh));
            const uint32_t v[2] = {q6k_code_bytes(L[2 * h + (q & 1)][0], H[h][0], q),
                                   q6k_code_bytes(L[2 * h + (q & 1)][1], H[h][1], q)};
            uint32_t bh[4], bl[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float p0 = sbyte(v[k >> 1], 2 * (k & 1)) * sc;       // exact: <= 15 bits
                const float p1 = sbyte(v[k >> 1], 2 * (k & 1) + 1) * sc;
                bh[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
                const float h0 = __builtin_bit_cast(float, bh[k] << 16);
                const float h1 = __builtin_bit_cast(float, bh[k] & 0xffff0000u);
                bl[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0 - h0, p1 - h1}, bf16x2));
            }
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(a_base + (cb + J) * 16);
            dsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bh), dsum, 0, 0, 0);
            dsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bl), dsum, 0, 0, 0);
        });
        const float d4 = half_bits_to_float(w.dh) * 0.25f;   // exact
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(d4, dsum[i], acc[i]);
        if (nig == ipg - 1) {
            // tile group done: partials of every wave through the slots
            const int it = blockIdx.x + (n / ipg) * gridDim.x;
            __syncthreads();
            *reinterpret_cast<f32x4*>(slot + (r * 20 + 4 * g) * 4) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            __syncthreads();
            const int outs = TPI * 16 * B;
            for (int t = tid; t < outs; t += 64 * NW) {
                const int tsl = t / (16 * B), rem = t % (16 * B), b = rem >> 4, rr = rem & 15;
                const int row = 16 * (it * TPI + tsl) + rr;
                float v = 0.f;
                for (int q = 0; q < KP; ++q) {
                    const float* pw = reinterpret_cast<const float*>(slots + (tsl * KP + q) * kSlot) + rr * 20;
                    v += pw[b];
                    v += pw[B + b];
                }
                if (row < N) y[b * ldy + row] = v;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = 0.f;
        }
    };

    // Two register buffers: the next item's loads are in flight while an
    // item is computed.
    if (total == 0) return;
    Q6KLane buf[2];
    load(0, buf[0]);
    for (int n = 0; n < total; n += 2) {
        load(n + 1, buf[1]);
        __builtin_amdgcn_sched_barrier(0);
        item(n, buf[0]);
        if (n + 1 >= total) break;
        load(n + 2, buf[0]);
        __builtin_amdgcn_sched_barrier(0);
        item(n + 1, buf[1]);
    }
}

template <int NW, class XT>
bool launch_q6k_mma(const uint8_t* W, int64_t N, int nsb, const XT* x, int64_t ldx, int B, float* y, int64_t ldy,
                    hipStream_t st, int kp_force, int32_t* rc) {
    constexpr int kSlot = 16 * 20 * 4;
    const size_t fixed = (size_t)NW * kSlot;
    const size_t per_blk = 128 * (size_t)B;             // staged pieces per 32-weight block
    if (fixed + 9 * per_blk > (size_t)kLdsMax) return false;
    const int64_t tiles = (N + 15) / 16;
    const int cus = device_cu_count();
    int KP = 1;
    if (kp_force > 0) {
        KP = kp_force;
        if (NW % KP || nsb % KP) return false;
    } else {
        while (KP < NW && nsb % (2 * KP) == 0 && (tiles + NW / KP - 1) / (NW / KP) < cus) KP *= 2;
    }
    // super-blocks per chunk: a multiple of KP
    int cs_max = 0;
    for (;; KP /= 2) {
        cs_max = (int)((kLdsMax - fixed) / per_blk - 1) / 8 / KP * KP;
        if (cs_max >= KP) break;
        if (KP == 1) return false;
    }
    const int nchunks = (nsb + cs_max - 1) / cs_max;
    const int cs = ((nsb + nchunks - 1) / nchunks + KP - 1) / KP * KP;
    const int KC = cs * 8;
    const size_t lds = fixed + (size_t)(KC | 1) * per_blk;

    auto kern = q6k_mma_kernel<NW, XT>;
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv", &dyn_max)) {
        *rc = e;
        return true;
    }
    if (lds > dyn_max) {
        *rc = fail(QMV_EINVAL, "qmv: %zu bytes of staged activations exceed the LDS", lds);
        return true;
    }
    const int64_t ngroups = (tiles + NW / KP - 1) / (NW / KP);
    const int per_cu = resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds);
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ngroups, (int64_t)cus * per_cu));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, W, (int)N, nsb, x, ldx, B, y, ldy, KP, KC);
    *rc = check_launch("qmv");
    return true;
}

template <class XT>
bool launch_q6k_mma_auto(const uint8_t* W, int64_t N, int nsb, const XT* x, int64_t ldx, int B, float* y,
                         int64_t ldy, hipStream_t st, int variant, int32_t* rc) {
    if (!aligned(x, XIn<XT>::kVecAlign)) return false;
    const int nw = (variant >> 8) == 16 ? 16 : 8;
    const int kp = variant & 0xff;
    return nw == 16 ? launch_q6k_mma<16, XT>(W, N, nsb, x, ldx, B, y, ldy, st, kp, rc)
                    : launch_q6k_mma<8, XT>(W, N, nsb, x, ldx, B, y, ldy, st, kp, rc);
}

}  // namespace

// Measured on the 8B decode shapes.  32-weight block formats, GPU time per
// launch from graph replays over cache-cold copies: the FMA kernels win at
// batch 2 except on the 128256-row lm_head (Q4_0 k / o / qkv / gate_up /
// down 4.5 / 6.1 / 7.5 / 23.3 / 15.8 us against 7.1 / 7.6 / 10.3 / 25.4 /
// 15.8), and at batch 3..4 on the 1024-row k and v, where every workgroup
// of the matrix-core kernel stages the whole activation block for a few
// row tiles (Q4_0 batch 3 5.4 against 7.6 us); from batch 5 and on larger
// matrices the matrix cores win or tie (batch 8 k 9.7 against 10.9, gate_up
// 26.4 against 53.2; Q8_0 and Q4_1 alike).  Whole steps (graph replays,
// same box, alternated twice) against the matrix cores from batch 2 (Q4_0)
// or 3: batch 2 +7% (Q4_0), batch 3 +5% (Q4_0) and +6% (Q4_1), batch 4 +4%
// (Q4_0, Q8_0), the row-fused steps unchanged; the FMA kernels on the
// 4096-row q and o as well lost 0.6-6% at batch 3..4.  The super-block
// formats' FMA kernels hold out longer (their matrix-core operands decode
// 6-bit fields and a pivot, or split scaled codes in two); per shape from
// graph replays, Q4_K / Q6_K: k (1024 rows) on the FMA kernels at every
// batch (batch 8 10.8 / 10.6 us against 11.1 / 12.5), 4096..6144 rows up
// to batch 5, 14336 and 28672 rows up to batch 3 (Q4_K) or 4 (Q6_K; Q4_K
// gate_up at batch 3 / 4 30.6 / 35.8 against 32.7 / 33.6), and
// 14336-column rows at batch 2 only (Q6_K down at batch 2 / 3 19.6 / 32.0
// against 28.2 / 27.9).  Whole steps against the earlier rule (matrix cores from batch
// 5, on long rows from batch 3): Q4_K batch 4 +3%, row-fused +8%, batch 5
// +1%; Q6_K batch 5 / 8 +3% / +2.5%; the rest unchanged.
bool use_mfma(qmv_fmt fmt, int64_t N, int nb, int B) {
    if (fmt == QMV_Q4_K || fmt == QMV_Q6_K) {
        if (N >= 65536) return B >= 2;
        if (nb >= 256) return B >= 3;
        if (N <= 1024) return false;
        if (N <= 6144) return B >= 6;
        return B >= (fmt == QMV_Q4_K ? 4 : 5);
    }
    if (N >= 65536) return B >= 2;
    if (B == 2) return false;
    if (B <= 4) return N > 1024 || nb >= 256;
    return true;
}

namespace {
// 16 waves per workgroup pay off on many tiles at batch 3..4 (the staged
// activations leave room for 16 slots) and on very many tiles above that;
// otherwise 8 (more tile groups than compute units, one activation chunk).
template <class F, class XT>
bool launch_mma_auto(const uint8_t* W, int64_t N, int nb, const XT* x, int64_t ldx, int B, float* y,
                     int64_t ldy, hipStream_t st, int variant, int32_t* rc) {
    if (!aligned(x, XIn<XT>::kVecAlign)) return false;
    const int64_t tiles = (N + 15) / 16;
    int nw = variant >> 8;
    if (nw == 0) nw = ((B >= 3 && B <= 4 && tiles >= 1024) || (B >= 5 && tiles >= 4096)) ? 16 : 8;
    const int kp = variant & 0xff;
    return nw == 16 ? launch_mma<F, 16, 8, 2, XT>(W, N, nb, x, ldx, B, y, ldy, st, kp, rc)
                    : launch_mma<F, 8, 8, 2, XT>(W, N, nb, x, ldx, B, y, ldy, st, kp, rc);
}

template <class F>
bool launch_mma_x(const uint8_t* W, int64_t N, int nb, const void* x, int32_t x_type, int64_t ldx, int B, float* y,
                  int64_t ldy, hipStream_t st, int variant, int32_t* rc) {
    switch (x_type) {
    case QMV_X_F32:
        return launch_mma_auto<F, float>(W, N, nb, static_cast<const float*>(x), ldx, B, y, ldy, st, variant, rc);
    case QMV_X_F16:
        return launch_mma_auto<F, _Float16>(W, N, nb, static_cast<const _Float16*>(x), ldx, B, y, ldy, st, variant,
                                            rc);
    case QMV_X_BF16:
        return launch_mma_auto<F, __bf16>(W, N, nb, static_cast<const __bf16*>(x), ldx, B, y, ldy, st, variant, rc);
    }
    return false;
}
}  // namespace

bool batch_matvec_mma(qmv_fmt fmt, const uint8_t* W, int64_t N, int nb, const void* x, int32_t x_type, int64_t ldx,
                      int B, float* y, int64_t ldy, hipStream_t st, int variant, int32_t* rc) {
    if (fmt == QMV_Q6_K) {
        const int nsb = nb / 8;
        if (B < 2 || B > 8 || nb % 8 || N > (1 << 30) || !aligned(W, 4) || ldx % 4) return false;
        switch (x_type) {
        case QMV_X_F32:
            return launch_q6k_mma_auto(W, N, nsb, static_cast<const float*>(x), ldx, B, y, ldy, st, variant, rc);
        case QMV_X_F16:
            return launch_q6k_mma_auto(W, N, nsb, static_cast<const _Float16*>(x), ldx, B, y, ldy, st, variant, rc);
        case QMV_X_BF16:
            return launch_q6k_mma_auto(W, N, nsb, static_cast<const __bf16*>(x), ldx, B, y, ldy, st, variant, rc);
        default: return false;
        }
    }
    const int64_t pitch = (int64_t)nb * (fmt == QMV_Q8_0 ? 34 : (fmt == QMV_Q4_1 ? 20 : 18));   // Q4_0, Q4_K: 18
    if (B < 2 || B > 8 || nb % 8 || N > (1 << 30) || pitch >= (1 << 24) || !aligned(W, 16) || ldx % 4) return false;
    switch (fmt) {
    case QMV_Q8_0: return launch_mma_x<Q8_0>(W, N, nb, x, x_type, ldx, B, y, ldy, st, variant, rc);
    case QMV_Q4_0: return launch_mma_x<Q4_0>(W, N, nb, x, x_type, ldx, B, y, ldy, st, variant, rc);
    case QMV_Q4_1: return launch_mma_x<Q4_1>(W, N, nb, x, x_type, ldx, B, y, ldy, st, variant, rc);
    case QMV_Q4_K: return launch_mma_x<Q4KSuper>(W, N, nb, x, x_type, ldx, B, y, ldy, st, variant, rc);
    default: return false;
    }
}

}  // namespace qmv
