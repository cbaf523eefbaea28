// Block-quantized (Q8_0 / Q4_0 / Q4_1) matrix x vector kernels for gfx950.
//
// What is computed: y[b][i] = sum_j DEQ(W)[i][j] * x[b][j], the decode-time
// matvec of "One Native Stack for Private, Continuously-Learning AI"
// (Sec. "The Unified Quant Core" and the QLoRA Lemma) that "Economical
// Serving and the hanzo.ai Platform" (Sec. 2.1) prices as one stream of the
// weights per token.  Like the pages' core, one kernel body serves every
// format; a per-format decoder turns a stored block into values in
// registers (Sec. 2.2 of the second page: block decoder + traits record).
//
// How it maps onto an MI355X (design notes, not taken from the pages):
//  * Lane-per-block.  Rows are split into segments of LPR lanes; lane li
//    of a segment handles blocks li, li+LPR, ... of its row, so the lanes of
//    a segment read consecutive blocks and a wave reads a contiguous run of
//    the row.  Blocks are 34/18/20 bytes, so each lane issues 4-byte-aligned
//    16-byte loads plus one 2-byte load, chosen so that no byte outside the
//    block is read (no over-read past the last block), and re-aligns the
//    codes in registers with v_alignbyte.  Weight loads are ordinary cached
//    loads: a 64-byte line is shared by neighbouring lanes and by the three
//    loads of a block, and a non-temporal hint (measured) loses a third of
//    the bandwidth to refetches.
//  * The activation vector is the only thing staged in LDS: x[b] once per
//    workgroup, padded to 36 floats per 32-block so that the 16-byte LDS
//    reads of neighbouring lanes fall in different banks, plus the per-block
//    sums sum_j x_j that fold the Q4_0 offset (-8) and the Q4_1 minimum m
//    into one multiply-add per block.
//  * Each lane accumulates RPL rows x B columns in fp32; a segment then
//    reduces across its LPR lanes with cross-lane shuffles in a fixed order
//    (deterministic, no atomics).
//  * No MFMA: at batch 1..8 this is a GEMV, bound by HBM bandwidth.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <cstdint>

#include "qmv_host.h"

namespace qmv {
namespace {

constexpr int kWaves = 4;               // waves per workgroup
constexpr int kThreads = 64 * kWaves;   // workgroup size
constexpr int kXPad = 36;               // floats per staged 32-block of x
constexpr int kLdsMax = 160 * 1024;     // LDS per workgroup on gfx950

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// --------------------------------------------------------------- loads
// p is 4-byte aligned; the hardware allows dword-aligned 16-byte loads.
__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4_a4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ uint32_t ld2(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(h & 0xffffu)));
}

// --------------------------------------------------------------- formats
// Traits + decoder per format.  load() fetches block g (global block index,
// row * blocks_per_row + column block) and leaves the scale(s) as floats and
// the code bytes 4-byte aligned in c[]:
//   Q8_0: c[0..7] = q_0..q_31 (int8, element 4i+k in byte k of c[i])
//   Q4_0/Q4_1: c[0..3] = qs[0..15] (low nibble of byte k of c[i] is element
//   4i+k, high nibble element 16+4i+k).
//
// fetch() only issues the loads into a Raw record; decode() turns the raw
// registers into the scale(s) and aligned codes.  Keeping them apart lets a
// wave have the next blocks in flight while it computes the current ones.
struct Q8_0 {
    static constexpr int kBytes = 34;
    static constexpr bool kNeedSx = false;   // the block term needs no sum of x
    struct Raw {
        u32x4 a, b;
        uint32_t u;
        uint32_t sh;
    };
    // 34g = 2g (mod 4): even blocks start 4-aligned (read [o, o+32) and the
    // last 2 code bytes), odd blocks start at 2 (mod 4) (read d alone, then
    // the 32 codes from o+2, 4-aligned).  Exactly the block's 34 bytes.
    __device__ static void fetch(const uint8_t* W, int64_t g, Raw& r) {
        const int64_t o = 34 * g;
        const bool even = (g & 1) == 0;
        r.a = ld16(W + o + (even ? 0 : 2));
        r.b = ld16(W + o + (even ? 16 : 18));
        r.u = ld2(W + o + (even ? 32 : 0));
        r.sh = even ? 2u : 0u;
    }
    __device__ static void decode(const Raw& r, float& d, float& m, uint32_t (&c)[8]) {
        const uint32_t w[9] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w, r.u};
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], r.sh);
        d = half_bits_to_float(r.sh ? r.a.x : r.u);
        m = 0.f;
    }
};

struct Q4_0 {
    static constexpr int kBytes = 18;
    static constexpr bool kNeedSx = true;    // folds the -8 offset
    struct Raw {
        u32x4 a;
        uint32_t u;
        uint32_t sh;
    };
    __device__ static void fetch(const uint8_t* W, int64_t g, Raw& r) {
        const int64_t o = 18 * g;
        const bool even = (g & 1) == 0;    // 18g = 2g (mod 4)
        r.a = ld16(W + o + (even ? 0 : 2));
        r.u = ld2(W + o + (even ? 16 : 0));
        r.sh = even ? 2u : 0u;
    }
    __device__ static void decode(const Raw& r, float& d, float& m, uint32_t (&c)[8]) {
        const uint32_t w[5] = {r.a.x, r.a.y, r.a.z, r.a.w, r.u};
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], r.sh);
        d = half_bits_to_float(r.sh ? r.a.x : r.u);
        m = 0.f;
    }
};

struct Q4_1 {
    static constexpr int kBytes = 20;
    static constexpr bool kNeedSx = true;    // folds the minimum m
    struct Raw {
        uint32_t dm;
        u32x4 a;
    };
    __device__ static void fetch(const uint8_t* W, int64_t g, Raw& r) {
        const int64_t o = 20 * g;          // always 4-aligned
        r.dm = ld4(W + o);
        r.a = ld16(W + o + 4);
    }
    __device__ static void decode(const Raw& r, float& d, float& m, uint32_t (&c)[8]) {
        c[0] = r.a.x; c[1] = r.a.y; c[2] = r.a.z; c[3] = r.a.w;
        d = half_bits_to_float(r.dm);
        m = half_bits_to_float(r.dm >> 16);
    }
};

// fetch + decode in one go (dequant kernel).
template <class F>
__device__ __forceinline__ void load_block(const uint8_t* W, int64_t g, float& d, float& m, uint32_t (&c)[8]) {
    typename F::Raw r;
    F::fetch(W, g, r);
    F::decode(r, d, m, c);
}

__device__ __forceinline__ float sbyte(uint32_t w, int k) {
    return static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(w >> (8 * k))));
}
__device__ __forceinline__ float ubyte(uint32_t w, int k) {
    return static_cast<float>((w >> (8 * k)) & 0xffu);
}

// Decoded element e of a block as float (the codes, before the scale).
// Used by the dequant kernel; the matvec kernel inlines the same steps.
template <class F>
__device__ __forceinline__ void block_values(const float d, const float m, const uint32_t (&c)[8], float (&v)[32]);

template <>
__device__ __forceinline__ void block_values<Q8_0>(const float d, const float, const uint32_t (&c)[8], float (&v)[32]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[4 * i + k] = d * sbyte(c[i], k);
}
template <>
__device__ __forceinline__ void block_values<Q4_0>(const float d, const float, const uint32_t (&c)[8], float (&v)[32]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = c[i] & 0x0f0f0f0fu, hi = (c[i] >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[4 * i + k] = d * (ubyte(lo, k) - 8.f);
            v[16 + 4 * i + k] = d * (ubyte(hi, k) - 8.f);
        }
    }
}
template <>
__device__ __forceinline__ void block_values<Q4_1>(const float d, const float m, const uint32_t (&c)[8], float (&v)[32]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = c[i] & 0x0f0f0f0fu, hi = (c[i] >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[4 * i + k] = __builtin_fmaf(d, ubyte(lo, k), m);
            v[16 + 4 * i + k] = __builtin_fmaf(d, ubyte(hi, k), m);
        }
    }
}

// The block's 32 codes as floats in element order: Q8_0 the signed bytes,
// Q4_0/Q4_1 the unsigned nibbles (offset and minimum are applied per block).
template <class F>
__device__ __forceinline__ void codes_to_float(const uint32_t (&c)[8], float (&q)[32]);

template <>
__device__ __forceinline__ void codes_to_float<Q8_0>(const uint32_t (&c)[8], float (&q)[32]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) q[4 * i + k] = sbyte(c[i], k);
}
__device__ __forceinline__ void nibbles_to_float(const uint32_t (&c)[8], float (&q)[32]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = c[i] & 0x0f0f0f0fu, hi = (c[i] >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            q[4 * i + k] = ubyte(lo, k);
            q[16 + 4 * i + k] = ubyte(hi, k);
        }
    }
}
template <>
__device__ __forceinline__ void codes_to_float<Q4_0>(const uint32_t (&c)[8], float (&q)[32]) { nibbles_to_float(c, q); }
template <>
__device__ __forceinline__ void codes_to_float<Q4_1>(const uint32_t (&c)[8], float (&q)[32]) { nibbles_to_float(c, q); }

// s[b] = sum_{e<32} q[e] * x_b[e] for the first w of B columns (w is
// wave-uniform: inactive columns are skipped by a scalar branch).  xs points
// at the block's 32 staged floats of column 0; column b is xstride_b after.
template <int B>
__device__ __forceinline__ void dot_cols(const float (&q)[32], const float* __restrict__ xs, int xstride_b,
                                         float (&s)[B], int w) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
        if (b < w) {
            const float* xp = xs + b * xstride_b;
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 xv = *reinterpret_cast<const float4*>(xp + 4 * i);
                a = __builtin_fmaf(q[4 * i + 0], xv.x, a);
                a = __builtin_fmaf(q[4 * i + 1], xv.y, a);
                a = __builtin_fmaf(q[4 * i + 2], xv.z, a);
                a = __builtin_fmaf(q[4 * i + 3], xv.w, a);
            }
            s[b] = a;
        }
    }
}

// Adds a block's term to the running sum, from the code dot s and the block
// sum sx of x.  Written with explicit fused multiply-adds so that every entry
// point (dense, MoE, any batch width) rounds identically.
template <class F> struct Term;
template <> struct Term<Q8_0> {
    __device__ static float add(float acc, float d, float, float s, float) { return __builtin_fmaf(d, s, acc); }
};
template <> struct Term<Q4_0> {
    // sum_j d*(c_j - 8) x_j = d * (sum_j c_j x_j - 8 sum_j x_j)
    __device__ static float add(float acc, float d, float, float s, float sx) {
        return __builtin_fmaf(d, __builtin_fmaf(-8.f, sx, s), acc);
    }
};
template <> struct Term<Q4_1> {
    // sum_j (d*c_j + m) x_j = d * sum_j c_j x_j + m * sum_j x_j
    __device__ static float add(float acc, float d, float m, float s, float sx) {
        return __builtin_fmaf(d, s, __builtin_fmaf(m, sx, acc));
    }
};

// Sum over the LPR consecutive lanes of a segment, in a fixed order; the
// total is valid in the segment's first lane (for LPR <= 16 in every lane of
// the segment).  Within 16-lane rows the sum uses DPP lane swizzles (a few
// VALU cycles each): xor 1, xor 2, half-row mirror, row mirror.  Across rows
// the row totals are read as scalars.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_val(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
template <int LPR>
__device__ __forceinline__ float segment_sum(float v) {
    static_assert(LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "segment width");
    v += dpp_mov<0xB1>(v);     // quad_perm [1,0,3,2]: pairs
    v += dpp_mov<0x4E>(v);     // quad_perm [2,3,0,1]: quads
    v += dpp_mov<0x141>(v);    // row_half_mirror: 8 lanes
    if (LPR >= 16) v += dpp_mov<0x140>(v);   // row_mirror: 16 lanes
    if (LPR == 32) {
        const float a = lane_val(v, 0) + lane_val(v, 16);
        const float b = lane_val(v, 32) + lane_val(v, 48);
        v = (threadIdx.x & 32) ? b : a;
    } else if (LPR == 64) {
        v = (lane_val(v, 0) + lane_val(v, 16)) + (lane_val(v, 32) + lane_val(v, 48));
    }
    return v;
}

// Straight-line staging of one 16-byte-aligned activation column (batch 1):
// every thread issues XU float4 loads (indices clamped, so the count is a
// compile-time constant), and only later writes them to LDS.  With no loop
// the compiler can keep other loads issued in between in flight while it
// waits for these.
template <int XU, int NT>
struct XStage {
    float4 v[XU];
    __device__ __forceinline__ void load(const float* __restrict__ x, int K4) {
        const float4* src = reinterpret_cast<const float4*>(x);
#pragma unroll
        for (int u = 0; u < XU; ++u) v[u] = src[min((int)threadIdx.x + u * NT, K4 - 1)];
    }
    // Indices past the end are clamped like the loads: such a thread
    // writes the last chunk's own value to the last chunk's slot.
    __device__ __forceinline__ void store(float* xs, int K4) const {
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int e = 4 * min((int)threadIdx.x + u * NT, K4 - 1);
            *reinterpret_cast<float4*>(xs + (e >> 5) * kXPad + (e & 31)) = v[u];
        }
    }
};

// Per-block sums of the staged columns (formats that fold an offset).
template <int NT>
__device__ __forceinline__ void block_sums(const float* xs, float* sx, int count) {
    for (int t = threadIdx.x; t < count; t += NT) {
        const float4* p = reinterpret_cast<const float4*>(xs + t * kXPad);
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 v = p[i];
            acc += v.x; acc += v.y; acc += v.z; acc += v.w;
        }
        sx[t] = acc;
    }
}

// Stages the first w of the B activation columns xcol[b][0..32*nb) into
// LDS as xs[b][block][36] and, when the format needs them, the per-block
// sums into sx[b][block].  Loads are issued in batches of 4 per thread
// before any is used, so the staging costs a few memory round trips, not
// one per element.  vec: every column is 16-byte aligned (float4 loads).
// Ends with a barrier.
template <bool kNeedSx, int B, int NT>
__device__ __forceinline__ void stage_x_cols(const float* const (&xcol)[B], int nb, float* xs, float* sx, int w,
                                             bool vec) {
    const int K = nb * 32;
    const int tid = threadIdx.x;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        if (b < w) {
            float* dst = xs + b * nb * kXPad;
            if (vec) {
                const float4* src = reinterpret_cast<const float4*>(xcol[b]);
                const int K4 = K >> 2;
                auto put = [&](int c, const float4& v) {
                    const int e = 4 * c;
                    *reinterpret_cast<float4*>(dst + (e >> 5) * kXPad + (e & 31)) = v;
                };
                for (int c0 = tid; c0 < K4; c0 += 4 * NT) {
                    const int c1 = c0 + NT, c2 = c0 + 2 * NT, c3 = c0 + 3 * NT;
                    const float4 v0 = src[c0];
                    const float4 v1 = src[min(c1, K4 - 1)];
                    const float4 v2 = src[min(c2, K4 - 1)];
                    const float4 v3 = src[min(c3, K4 - 1)];
                    put(c0, v0);
                    if (c1 < K4) put(c1, v1);
                    if (c2 < K4) put(c2, v2);
                    if (c3 < K4) put(c3, v3);
                }
            } else {
                const float* src = xcol[b];
                auto put = [&](int e, float v) { dst[(e >> 5) * kXPad + (e & 31)] = v; };
                for (int e0 = tid; e0 < K; e0 += 4 * NT) {
                    const int e1 = e0 + NT, e2 = e0 + 2 * NT, e3 = e0 + 3 * NT;
                    const float v0 = src[e0];
                    const float v1 = src[min(e1, K - 1)];
                    const float v2 = src[min(e2, K - 1)];
                    const float v3 = src[min(e3, K - 1)];
                    put(e0, v0);
                    if (e1 < K) put(e1, v1);
                    if (e2 < K) put(e2, v2);
                    if (e3 < K) put(e3, v3);
                }
            }
        }
    }
    __syncthreads();
    if (kNeedSx) {
        block_sums<NT>(xs, sx, w * nb);
        __syncthreads();
    }
}

// ------------------------------------------------------------------ kernels
// Computes, for the rows row0 + r*G + seg (r < RPL) of an N-row matrix with
// nb blocks per row, the B dot products with the staged activations, and
// leaves the segment totals in acc (identical in all LPR lanes).
template <class F, int B, int LPR, int RPL>
__device__ __forceinline__ void tile_rows(const uint8_t* __restrict__ W, int64_t N, int nb, int64_t row0,
                                          const float* __restrict__ xs, const float* __restrict__ sx,
                                          float (&acc)[RPL][B], int w) {
    constexpr int G = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int xb = nb * kXPad;
    int64_t gbase[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int64_t row = row0 + r * G + seg;
        gbase[r] = (row < N ? row : N - 1) * nb;   // clamp: loads stay in bounds
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.f;

    for (int j = li; j < nb; j += LPR) {
        float d[RPL], m[RPL];
        uint32_t c[RPL][8];
#pragma unroll
        for (int r = 0; r < RPL; ++r) load_block<F>(W, gbase[r] + j, d[r], m[r], c[r]);
        const float* xj = xs + j * kXPad;
        float sxb[B];
#pragma unroll
        for (int b = 0; b < B; ++b) sxb[b] = b < w ? sx[b * nb + j] : 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            float q[32];
            codes_to_float<F>(c[r], q);
            float s[B];
#pragma unroll
            for (int b = 0; b < B; ++b) s[b] = 0.f;
            dot_cols<B>(q, xj, xb, s, w);
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = Term<F>::add(acc[r][b], d[r], m[r], s[b], sxb[b]);
        }
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = segment_sum<LPR>(acc[r][b]);
}

// Dense matvec.  A persistent grid (as many workgroups as fit on the GPU at
// once); wave w of the grid takes row tiles w, w + waves, ... .  A tile is
// G*RPL rows (G row segments of LPR lanes, RPL rows per lane) and is worked
// through in T = ceil(nb/LPR) steps; in step t lane li reads block
// li + LPR*t of each of its RPL rows.  The blocks of the next step are
// loaded while the current step is computed (two steps in flight per wave),
// and the first step's loads are issued before the activation staging so
// that both latencies overlap.
template <class F, int B, int LPR, int RPL, int XU, int NW>
__global__ __launch_bounds__(64 * NW) void qmv_kernel(const uint8_t* __restrict__ W, int64_t N, int nb,
                                                       const float* __restrict__ x, int64_t ldx,
                                                       float* __restrict__ y, int64_t ldy, int xvec) {
    extern __shared__ float lds[];
    float* xs = lds;
    float* sx = lds + B * nb * kXPad;

    constexpr int G = 64 / LPR;
    constexpr int ROWS = G * RPL;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int T = (nb + LPR - 1) / LPR;
    const int64_t ntiles = (N + ROWS - 1) / ROWS;
    const int64_t wstride = (int64_t)gridDim.x * NW;

    // Step (tile, t): lane li handles block li + LPR*t of its RPL rows.
    using Raw = typename F::Raw;
    auto load_step = [&](int64_t tile, int t, Raw (&blk)[RPL]) {
        const int j = min(li + LPR * t, nb - 1);      // clamp: stays in bounds
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int64_t row = min(tile * ROWS + r * G + seg, N - 1);
            F::fetch(W, row * nb + j, blk[r]);
        }
    };
    float acc[RPL][B];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.f;

    auto compute_step = [&](int64_t tile, int t, const Raw (&blk)[RPL]) {
        const int j = li + LPR * t;
        const bool valid = j < nb;
        const int jc = valid ? j : nb - 1;
        const float* xj = xs + jc * kXPad;
        float sxb[B];
#pragma unroll
        for (int b = 0; b < B; ++b) sxb[b] = F::kNeedSx ? sx[b * nb + jc] : 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            float d, m;
            uint32_t c[8];
            F::decode(blk[r], d, m, c);
            float q[32];
            codes_to_float<F>(c, q);
            float sdot[B];
#pragma unroll
            for (int b = 0; b < B; ++b) sdot[b] = 0.f;
            dot_cols<B>(q, xj, nb * kXPad, sdot, B);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float upd = Term<F>::add(acc[r][b], d, m, sdot[b], sxb[b]);
                acc[r][b] = valid ? upd : acc[r][b];
            }
        }
        if (t == T - 1) {   // tile done: reduce the segments and write
#pragma unroll
            for (int r = 0; r < RPL; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) acc[r][b] = segment_sum<LPR>(acc[r][b]);
            if (li == 0) {
#pragma unroll
                for (int r = 0; r < RPL; ++r) {
                    const int64_t row = tile * ROWS + r * G + seg;
                    if (row < N) {
#pragma unroll
                        for (int b = 0; b < B; ++b) y[b * ldy + row] = acc[r][b];
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RPL; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) acc[r][b] = 0.f;
        }
    };
    auto advance = [&](int64_t& tile, int& t) {
        if (++t == T) { t = 0; tile += wstride; }
    };

    // Two register buffers used in turn: the loads of one step are in flight
    // while the previous step is computed.  Loads are issued without
    // branches (a wave past its last step re-reads its current blocks, which
    // are in cache), so the compiler waits only for the buffer in use.
    int64_t tileA = (int64_t)blockIdx.x * NW + wave;
    int tA = 0;
    Raw bufA[RPL], bufB[RPL];
    const int K4 = nb * 8;
    if (XU > 0 && xvec) {
        // batch 1: x loads, then the first weight loads, then x into LDS
        XStage<XU, 64 * NW> xst;
        xst.load(x, K4);
        load_step(min(tileA, ntiles - 1), tA, bufA);
        __builtin_amdgcn_sched_barrier(0);   // keep both batches of loads issued first
        xst.store(xs, K4);
        __syncthreads();
        if (F::kNeedSx) {
            block_sums<64 * NW>(xs, sx, nb);
            __syncthreads();
        }
    } else {
        const float* xcol[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xcol[b] = x + b * ldx;
        stage_x_cols<F::kNeedSx, B, 64 * NW>(xcol, nb, xs, sx, B, xvec != 0);
        load_step(min(tileA, ntiles - 1), tA, bufA);
    }

    if (tileA < ntiles) {
        while (true) {
            int64_t tileB = tileA;
            int tB = tA;
            advance(tileB, tB);
            const bool hasB = tileB < ntiles;
            load_step(hasB ? tileB : tileA, hasB ? tB : tA, bufB);
            __builtin_amdgcn_sched_barrier(0);   // issue B's loads before using A
            compute_step(tileA, tA, bufA);
            if (!hasB) break;
            tileA = tileB;
            tA = tB;
            advance(tileA, tA);
            const bool hasA = tileA < ntiles;
            load_step(hasA ? tileA : tileB, hasA ? tA : tB, bufA);
            __builtin_amdgcn_sched_barrier(0);   // issue A's loads before using B
            compute_step(tileB, tB, bufB);
            if (!hasA) break;
        }
    }
}

// Grouped MoE expert matvec.  blockIdx.y = u selects the u-th distinct
// expert id in first-occurrence order of ids[0..P); the workgroup streams
// rows [blockIdx.x*ROWS_WG, +ROWS_WG) of that expert once per group of up
// to 8 (token, slot) pairs routed to it (one group in the usual case of
// distinct ids per token), in pair order.
constexpr int kMoeMaxPairs = 128;
constexpr int kMoeStaticLds = 4096;  // s_ids/s_first/s_members/scalars, rounded up

// One group of w <= 8 member pairs: stage their activations, then the
// wave's rows of the expert, written to each member's output rows.
template <class F, int LPR, int RPL>
__device__ __forceinline__ void moe_chunk(const uint8_t* __restrict__ We, int64_t N, int nb, int64_t wg_row0,
                                          const float* __restrict__ x, int64_t xs_tok, int64_t xs_slot, int top_k,
                                          const int* __restrict__ members, int w, float* __restrict__ y, float* xs,
                                          float* sx) {
    constexpr int B = 8;
    constexpr int G = 64 / LPR;
    constexpr int ROWS = G * RPL;
    const float* xcol[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const int p = b < w ? members[b] : 0;
        xcol[b] = x + (int64_t)(p / top_k) * xs_tok + (int64_t)(p % top_k) * xs_slot;
    }
    stage_x_cols<F::kNeedSx, B, kThreads>(xcol, nb, xs, sx, w, false);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int64_t row0 = wg_row0 + (int64_t)wave * ROWS;
    if (row0 < N) {
        float acc[RPL][B];
        tile_rows<F, B, LPR, RPL>(We, N, nb, row0, xs, sx, acc, w);
        if (li == 0) {
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int64_t row = row0 + r * G + seg;
                if (row < N) {
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        if (b < w) y[(int64_t)members[b] * N + row] = acc[r][b];
                }
            }
        }
    }
    __syncthreads();   // xs is restaged by the next group
}

template <class F, int LPR, int RPL>
__global__ __launch_bounds__(kThreads) void moe_kernel(const uint8_t* __restrict__ Wx, int64_t estride,
                                                       int n_experts, int64_t N, int nb,
                                                       const int32_t* __restrict__ ids, int P, int top_k,
                                                       const float* __restrict__ x, int64_t xs_tok,
                                                       int64_t xs_slot, float* __restrict__ y, int max_cols) {
    __shared__ int s_ids[kMoeMaxPairs];
    __shared__ int s_first[kMoeMaxPairs];
    __shared__ int s_members[kMoeMaxPairs];
    __shared__ int s_expert, s_has, s_nmem;
    extern __shared__ float lds[];
    const int t = threadIdx.x;
    const int u = blockIdx.y;
    if (t < P) s_ids[t] = ids[t];
    if (t == 0) { s_has = 0; s_nmem = 0; }
    __syncthreads();
    // first[t]: pair t carries the first occurrence of its id.
    if (t < P) {
        int f = 1;
        for (int q = 0; q < t; ++q) f &= (s_ids[q] != s_ids[t]) ? 1 : 0;
        s_first[t] = f;
    }
    __syncthreads();
    // The group index of a first occurrence is the number of first
    // occurrences before it.
    if (t < P && s_first[t]) {
        int rank = 0;
        for (int q = 0; q < t; ++q) rank += s_first[q];
        if (rank == u) { s_expert = s_ids[t]; s_has = 1; }
    }
    __syncthreads();
    if (!s_has) return;                       // fewer than u+1 distinct ids
    const int e = s_expert;
    if (t < P && s_ids[t] == e) {
        int pos = 0;
        for (int q = 0; q < t; ++q) pos += (s_ids[q] == e) ? 1 : 0;
        s_members[pos] = t;
        int after = 0;
        for (int q = t + 1; q < P; ++q) after += (s_ids[q] == e) ? 1 : 0;
        if (after == 0) s_nmem = pos + 1;     // the last member writes the count
    }
    __syncthreads();
    const int nmem = s_nmem;
    constexpr int ROWS_WG = kWaves * (64 / LPR) * RPL;
    const int64_t wg_row0 = (int64_t)blockIdx.x * ROWS_WG;
    if (e < 0 || e >= n_experts) {
        // An id outside [0, n_experts) cannot be reported to the host:
        // its outputs become quiet NaN.
        const float qnan = __builtin_nanf("");
        for (int k = 0; k < nmem; ++k)
            for (int64_t row = wg_row0 + t; row < wg_row0 + ROWS_WG && row < N; row += kThreads)
                y[(int64_t)s_members[k] * N + row] = qnan;
        return;
    }
    const uint8_t* We = Wx + (int64_t)e * estride;
    float* xs = lds;
    float* sx = lds + max_cols * nb * kXPad;
    for (int c0 = 0; c0 < nmem; c0 += max_cols) {
        const int w = min(max_cols, nmem - c0);
        moe_chunk<F, LPR, RPL>(We, N, nb, wg_row0, x, xs_tok, xs_slot, top_k, s_members + c0, w, y, xs, sx);
    }
}

// One thread per block: out[g*32 + e] = value e of block g.
template <class F>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ W, int64_t nblocks,
                                                           float* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= nblocks) return;
    float d, m;
    uint32_t c[8];
    load_block<F>(W, g, d, m, c);
    float v[32];
    block_values<F>(d, m, c, v);
    float* o = out + g * 32;
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = v[e];
}

// ------------------------------------------------------------------ host
constexpr int kRpl = 2;   // MoE rows per lane

template <class F, int B, int LPR, int XU, int NW>
int32_t launch_b(const uint8_t* W, int64_t N, int nb, const float* x, int64_t ldx, float* y, int64_t ldy,
                 hipStream_t st) {
    constexpr int RPL = 1;
    auto kern = qmv_kernel<F, B, LPR, RPL, XU, NW>;
    const size_t lds = (size_t)B * nb * (kXPad + (F::kNeedSx ? 1 : 0)) * sizeof(float);
    static bool attr_set = false;   // benign race: every thread sets the same value
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                kLdsMax) != hipSuccess)
            return fail(QMV_EHIP, "qmv: cannot raise the LDS limit: %s", hipGetErrorString(hipGetLastError()));
        attr_set = true;
    }
    constexpr int rows_per_wg = NW * (64 / LPR) * RPL;
    const int64_t tiles = (N + rows_per_wg - 1) / rows_per_wg;
    const int per_cu = resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds);
    const int64_t cap = (int64_t)device_cu_count() * per_cu;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, cap));
    const int xvec = (aligned(x, 16) && ldx % 4 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, W, N, nb, x, ldx, y, ldy, xvec);
    return check_launch("qmv");
}

// Lanes per row: whole waves for long rows, smaller segments for short rows
// so that lanes are not left idle (e.g. 24 blocks -> 8 lanes x 3).
template <class F, int B, int XU, int NW>
int32_t launch_lpr(const uint8_t* W, int64_t N, int nb, const float* x, int64_t ldx, float* y, int64_t ldy,
                   hipStream_t st) {
    if (nb >= 64) return launch_b<F, B, 64, XU, NW>(W, N, nb, x, ldx, y, ldy, st);
    if (nb >= 32) return launch_b<F, B, 32, XU, NW>(W, N, nb, x, ldx, y, ldy, st);
    return launch_b<F, B, 8, XU, NW>(W, N, nb, x, ldx, y, ldy, st);
}

// Batch 1.  Workgroups of 8 waves when the staged activations (> 40 KB)
// allow few workgroups per CU, else 4 (more, smaller workgroups spread
// small matrices over every CU).  Activations are staged with straight-line
// 16-byte loads when 16-byte aligned: XU loads per thread cover
// K <= 16 * 64 * NW * XU / 4.
template <class F>
int32_t launch_b1(const uint8_t* W, int64_t N, int nb, const float* x, int64_t ldx, float* y, int64_t ldy,
                  hipStream_t st) {
    const size_t lds = (size_t)nb * (kXPad + (F::kNeedSx ? 1 : 0)) * sizeof(float);
    const bool vec = aligned(x, 16);
    const int K4 = nb * 8;
    if (lds > 40 * 1024) {
        if (vec && K4 <= 2 * 512) return launch_lpr<F, 1, 2, 8>(W, N, nb, x, ldx, y, ldy, st);
        if (vec && K4 <= 8 * 512) return launch_lpr<F, 1, 8, 8>(W, N, nb, x, ldx, y, ldy, st);
        return launch_lpr<F, 1, 0, 8>(W, N, nb, x, ldx, y, ldy, st);
    }
    if (vec && K4 <= 4 * 256) return launch_lpr<F, 1, 4, 4>(W, N, nb, x, ldx, y, ldy, st);
    if (vec && K4 <= 16 * 256) return launch_lpr<F, 1, 16, 4>(W, N, nb, x, ldx, y, ldy, st);
    return launch_lpr<F, 1, 0, 4>(W, N, nb, x, ldx, y, ldy, st);
}

template <class F>
int32_t launch_batch(const uint8_t* W, int64_t N, int nb, const float* x, int64_t ldx, int B, float* y,
                     int64_t ldy, hipStream_t st) {
    switch (B) {
    case 1: return launch_b1<F>(W, N, nb, x, ldx, y, ldy, st);
    case 2: return launch_lpr<F, 2, 0, 8>(W, N, nb, x, ldx, y, ldy, st);
    case 3: return launch_lpr<F, 3, 0, 8>(W, N, nb, x, ldx, y, ldy, st);
    case 4: return launch_lpr<F, 4, 0, 8>(W, N, nb, x, ldx, y, ldy, st);
    case 5: return launch_lpr<F, 5, 0, 8>(W, N, nb, x, ldx, y, ldy, st);
    case 6: return launch_lpr<F, 6, 0, 8>(W, N, nb, x, ldx, y, ldy, st);
    case 7: return launch_lpr<F, 7, 0, 8>(W, N, nb, x, ldx, y, ldy, st);
    default: return launch_lpr<F, 8, 0, 8>(W, N, nb, x, ldx, y, ldy, st);
    }
}

int32_t check_common(const char* name, const void* W, int64_t N, int64_t K, const void* x, int64_t ldx,
                     int32_t batch, const void* y, int64_t ldy) {
    if (!W || !x || !y) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (N < 1) return fail(QMV_EINVAL, "%s: n_rows must be >= 1 (got %lld)", name, (long long)N);
    if (K < 32 || K % 32) return fail(QMV_EINVAL, "%s: n_cols must be a positive multiple of 32 (got %lld)", name, (long long)K);
    if (batch < 1 || batch > 8) return fail(QMV_EINVAL, "%s: batch must be in 1..8 (got %d)", name, batch);
    if (ldx < K) return fail(QMV_EINVAL, "%s: ldx (%lld) < n_cols (%lld)", name, (long long)ldx, (long long)K);
    if (ldy < N) return fail(QMV_EINVAL, "%s: ldy (%lld) < n_rows (%lld)", name, (long long)ldy, (long long)N);
    if (K / 32 > (1 << 26) || N > ((int64_t)1 << 40) / (K / 32))
        return fail(QMV_EINVAL, "%s: matrix too large (%lld x %lld)", name, (long long)N, (long long)K);
    if (!aligned(W, 4) || !aligned(x, 4) || !aligned(y, 4))
        return fail(QMV_EALIGN, "%s: W, x and y must be 4-byte aligned", name);
    return QMV_OK;
}

template <class F>
int32_t matvec(const char* name, const void* W, int64_t N, int64_t K, const float* x, int64_t ldx, int32_t batch,
               float* y, int64_t ldy, void* stream) {
    int32_t rc = check_common(name, W, N, K, x, ldx, batch, y, ldy);
    if (rc != QMV_OK) return rc;
    const int nb = (int)(K / 32);
    // The staged activation block must fit in LDS; wider batches than fit
    // are processed in column groups (each group re-reads W).
    const int per_col = nb * (kXPad + (F::kNeedSx ? 1 : 0)) * (int)sizeof(float);
    const int per_pass = std::max(1, std::min<int>(batch, kLdsMax / per_col));
    if (per_col > kLdsMax)
        return fail(QMV_EINVAL, "%s: n_cols %lld too large for one activation row in LDS", name, (long long)K);
    for (int b0 = 0; b0 < batch; b0 += per_pass) {
        const int bw = std::min(per_pass, batch - b0);
        rc = launch_batch<F>(static_cast<const uint8_t*>(W), N, nb, x + b0 * ldx, ldx, bw, y + b0 * ldy, ldy,
                             as_stream(stream));
        if (rc != QMV_OK) return rc;
    }
    return ok();
}

template <class F>
int32_t dequant(const void* W, int64_t N, int64_t K, float* out, void* stream) {
    int32_t rc = check_common("qmv_dequant", W, N, K, out, K, 1, out, N);
    if (rc != QMV_OK) return rc;
    const int64_t nblocks = N * (K / 32);
    const int64_t grid = (nblocks + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(dequant_kernel<F>, dim3((unsigned)grid), dim3(kThreads), 0, as_stream(stream),
                       static_cast<const uint8_t*>(W), nblocks, out);
    return check_launch("qmv_dequant");
}

template <class F, int LPR>
int32_t launch_moe_lpr(const uint8_t* Wx, int64_t estride, int n_experts, int64_t N, int nb, const int32_t* ids,
                       int P, int top_k, const float* x, int64_t xs_tok, int64_t xs_slot, float* y, int max_cols,
                       hipStream_t st) {
    auto kern = moe_kernel<F, LPR, kRpl>;
    static bool attr_set = false;   // benign race: every thread sets the same value
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                kLdsMax - kMoeStaticLds) != hipSuccess)
            return fail(QMV_EHIP, "qmv_moe: cannot raise the LDS limit: %s", hipGetErrorString(hipGetLastError()));
        attr_set = true;
    }
    constexpr int rows_per_wg = kWaves * (64 / LPR) * kRpl;
    const size_t lds = (size_t)max_cols * nb * (kXPad + 1) * sizeof(float);
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg), (unsigned)P);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, Wx, estride, n_experts, N, nb, ids, P, top_k, x, xs_tok,
                       xs_slot, y, max_cols);
    return check_launch("qmv_moe");
}

template <class F>
int32_t moe(const void* Wx, int64_t estride, int32_t n_experts, int64_t N, int64_t K, const int32_t* ids,
            int32_t batch, int32_t top_k, const float* x, int64_t xs_tok, int64_t xs_slot, float* y, void* stream) {
    const char* name = "qmv_moe";
    if (!Wx || !ids || !x || !y) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (n_experts < 1) return fail(QMV_EINVAL, "%s: n_experts must be >= 1", name);
    if (N < 1 || K < 32 || K % 32) return fail(QMV_EINVAL, "%s: bad matrix shape %lld x %lld", name, (long long)N, (long long)K);
    if (batch < 1 || batch > 8) return fail(QMV_EINVAL, "%s: batch must be in 1..8 (got %d)", name, batch);
    if (top_k < 1 || top_k > 16) return fail(QMV_EINVAL, "%s: top_k must be in 1..16 (got %d)", name, top_k);
    const int64_t nb = K / 32;
    if (nb > (1 << 26) || N > ((int64_t)1 << 40) / nb) return fail(QMV_EINVAL, "%s: matrix too large", name);
    const int64_t mbytes = N * nb * F::kBytes;
    if (estride < mbytes || estride % 4)
        return fail(QMV_EINVAL, "%s: expert_stride_bytes (%lld) must be >= %lld and a multiple of 4", name,
                    (long long)estride, (long long)mbytes);
    if (n_experts > 1 && estride > ((int64_t)1 << 46) / (n_experts - 1)) return fail(QMV_EINVAL, "%s: experts too large", name);
    if (batch > 1 && xs_tok < K) return fail(QMV_EINVAL, "%s: x_stride_token must be >= n_cols", name);
    if (xs_tok < 0) return fail(QMV_EINVAL, "%s: x_stride_token must be >= 0", name);
    if (top_k > 1 && xs_slot != 0 && xs_slot < K) return fail(QMV_EINVAL, "%s: x_stride_slot must be 0 or >= n_cols", name);
    if (xs_slot < 0) return fail(QMV_EINVAL, "%s: x_stride_slot must be >= 0", name);
    if (!aligned(Wx, 4) || !aligned(x, 4) || !aligned(y, 4) || !aligned(ids, 4))
        return fail(QMV_EALIGN, "%s: W_experts, x, y and expert_ids must be 4-byte aligned", name);
    const int64_t per_col = nb * (kXPad + 1) * (int64_t)sizeof(float);
    const int max_cols = (int)std::min<int64_t>(8, (kLdsMax - kMoeStaticLds) / per_col);
    if (max_cols < 1) return fail(QMV_EINVAL, "%s: n_cols %lld too large for one activation row in LDS", name, (long long)K);
    const int P = batch * top_k;
    const uint8_t* W8 = static_cast<const uint8_t*>(Wx);
    hipStream_t st = as_stream(stream);
    if (nb >= 64) return launch_moe_lpr<F, 64>(W8, estride, n_experts, N, (int)nb, ids, P, top_k, x, xs_tok, xs_slot, y, max_cols, st);
    if (nb >= 32) return launch_moe_lpr<F, 32>(W8, estride, n_experts, N, (int)nb, ids, P, top_k, x, xs_tok, xs_slot, y, max_cols, st);
    return launch_moe_lpr<F, 8>(W8, estride, n_experts, N, (int)nb, ids, P, top_k, x, xs_tok, xs_slot, y, max_cols, st);
}

}  // namespace
}  // namespace qmv

extern "C" int32_t qmv_q8_0(const void* W, int64_t n_rows, int64_t n_cols, const float* x, int64_t ldx, int32_t batch,
                            float* y, int64_t ldy, void* stream) {
    return qmv::matvec<qmv::Q8_0>("qmv_q8_0", W, n_rows, n_cols, x, ldx, batch, y, ldy, stream);
}
extern "C" int32_t qmv_q4_0(const void* W, int64_t n_rows, int64_t n_cols, const float* x, int64_t ldx, int32_t batch,
                            float* y, int64_t ldy, void* stream) {
    return qmv::matvec<qmv::Q4_0>("qmv_q4_0", W, n_rows, n_cols, x, ldx, batch, y, ldy, stream);
}
extern "C" int32_t qmv_q4_1(const void* W, int64_t n_rows, int64_t n_cols, const float* x, int64_t ldx, int32_t batch,
                            float* y, int64_t ldy, void* stream) {
    return qmv::matvec<qmv::Q4_1>("qmv_q4_1", W, n_rows, n_cols, x, ldx, batch, y, ldy, stream);
}
extern "C" int32_t qmv_dequant(qmv_fmt fmt, const void* W, int64_t n_rows, int64_t n_cols, float* out, void* stream) {
    switch (fmt) {
    case QMV_Q8_0: return qmv::dequant<qmv::Q8_0>(W, n_rows, n_cols, out, stream);
    case QMV_Q4_0: return qmv::dequant<qmv::Q4_0>(W, n_rows, n_cols, out, stream);
    case QMV_Q4_1: return qmv::dequant<qmv::Q4_1>(W, n_rows, n_cols, out, stream);
    default: return qmv::fail(QMV_EUNSUPPORTED, "qmv_dequant: unknown format %d", (int)fmt);
    }
}
extern "C" int32_t qmv_moe(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes, int32_t n_experts,
                           int64_t n_rows, int64_t n_cols, const int32_t* expert_ids, int32_t batch, int32_t top_k,
                           const float* x, int64_t x_stride_token, int64_t x_stride_slot, float* y, void* stream) {
    switch (fmt) {
    case QMV_Q8_0:
        return qmv::moe<qmv::Q8_0>(W_experts, expert_stride_bytes, n_experts, n_rows, n_cols, expert_ids, batch, top_k,
                                   x, x_stride_token, x_stride_slot, y, stream);
    case QMV_Q4_0:
        return qmv::moe<qmv::Q4_0>(W_experts, expert_stride_bytes, n_experts, n_rows, n_cols, expert_ids, batch, top_k,
                                   x, x_stride_token, x_stride_slot, y, stream);
    case QMV_Q4_1:
        return qmv::moe<qmv::Q4_1>(W_experts, expert_stride_bytes, n_experts, n_rows, n_cols, expert_ids, batch, top_k,
                                   x, x_stride_token, x_stride_slot, y, stream);
    default: return qmv::fail(QMV_EUNSUPPORTED, "qmv_moe: unknown format %d", (int)fmt);
    }
}
