// Device building blocks shared by the block-format kernels: per-format
// block fetch/decode, code conversion, the block dot product and term, the
// segment reduction and the activation staging.  Included by each kernel
// translation unit (everything is in an anonymous namespace).
//
// Accuracy: every block term is formed so that its rounding error is
// relative to sum_j |w_j x_j| of the block, whatever the codes: Q8_0 and
// Q4_0 dot signed codes (c - 8 for Q4_0) with x and scale the block dot by
// d; Q4_1 dequantizes each weight (d*c + m, exact in fp32 for stored
// blocks whose value bits span <= 24) before the dot.  No term subtracts
// two sums of |x| size, which would cancel on rows of zero weights.
#pragma once
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

constexpr int kPolicyNT = 2;               // buffer-load cache policy: non-temporal
constexpr int kRawBufferFlags = 0x00020000;   // descriptor word 3 of a raw (untyped) buffer

// A raw buffer descriptor over [p, p + bytes), bytes < 2^32.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kRawBufferFlags);
}

// --------------------------------------------------------------- loads
// p is 4-byte aligned; the hardware allows dword-aligned 16-byte loads.
__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4_a4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ uint32_t ld2(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(h & 0xffffu)));
}

// --------------------------------------------------------------- activations
// Activation element types: fp32, fp16 (_Float16) and bf16 (__bf16).  Staging
// widens 16-bit activations to fp32 exactly, so every kernel computes on the
// same fp32 values an fp32 call with the widened activations would.
// load4: elements p[0..3] (p aligned to kVecAlign); load1: p[0].
template <class XT> struct XIn;
template <> struct XIn<float> {
    static constexpr int kVecAlign = 16;
    __device__ static float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ static float load1(const float* p) { return *p; }
};
template <> struct XIn<_Float16> {
    static constexpr int kVecAlign = 8;
    __device__ static float4 load4(const _Float16* p) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        return float4{half_bits_to_float(w.x), half_bits_to_float(w.x >> 16), half_bits_to_float(w.y),
                      half_bits_to_float(w.y >> 16)};
    }
    __device__ static float load1(const _Float16* p) {
        return half_bits_to_float(*reinterpret_cast<const uint16_t*>(p));
    }
};
template <> struct XIn<__bf16> {
    static constexpr int kVecAlign = 8;
    __device__ static float bits(uint32_t hi16) { return __builtin_bit_cast(float, hi16); }
    __device__ static float4 load4(const __bf16* p) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        return float4{bits(w.x << 16), bits(w.x & 0xffff0000u), bits(w.y << 16), bits(w.y & 0xffff0000u)};
    }
    __device__ static float load1(const __bf16* p) {
        return bits((uint32_t)*reinterpret_cast<const uint16_t*>(p) << 16);
    }
};

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
    static constexpr bool kNibbles = false;  // 8-bit codes
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
    // Block l of a step of 64 blocks copied to LDS at s (16-byte aligned):
    // the same registers fetch() leaves for a block of the same parity.
    __device__ static void from_lds(const uint8_t* s, int l, Raw& r) {
        const int o = 34 * l;
        const bool even = (l & 1) == 0;
        const uint32_t* a = reinterpret_cast<const uint32_t*>(s + o + (even ? 0 : 2));
        r.a = u32x4{a[0], a[1], a[2], a[3]};
        r.b = u32x4{a[4], a[5], a[6], a[7]};
        r.u = *reinterpret_cast<const uint32_t*>(s + (even ? o + 32 : o - 2)) >> (even ? 0 : 16);
        r.sh = even ? 2u : 0u;
    }
};

struct Q4_0 {
    static constexpr int kBytes = 18;
    static constexpr bool kNibbles = true;   // 4-bit codes
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
    __device__ static void from_lds(const uint8_t* s, int l, Raw& r) {
        const int o = 18 * l;
        const bool even = (l & 1) == 0;
        const uint32_t* a = reinterpret_cast<const uint32_t*>(s + o + (even ? 0 : 2));
        r.a = u32x4{a[0], a[1], a[2], a[3]};
        r.u = *reinterpret_cast<const uint32_t*>(s + (even ? o + 16 : o - 2)) >> (even ? 0 : 16);
        r.sh = even ? 2u : 0u;
    }
};

struct Q4_1 {
    static constexpr int kBytes = 20;
    static constexpr bool kNibbles = true;   // 4-bit codes
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
    __device__ static void from_lds(const uint8_t* s, int l, Raw& r) {
        const uint32_t* a = reinterpret_cast<const uint32_t*>(s + 20 * l);
        r.dm = a[0];
        r.a = u32x4{a[1], a[2], a[3], a[4]};
    }
};

// A step of 64 consecutive blocks read as whole 16-byte chunks: lane l
// loads chunks l, 64 + l, ... (lanes past the last chunk re-read it, so
// every load is in bounds and branch-free).  Each load instruction covers
// whole cache lines, which lets the weights stream with non-temporal loads.
template <class F>
struct Contig {
    static constexpr int kStepBytes = 64 * F::kBytes;        // 2176 / 1152 / 1280
    static constexpr int kChunks = kStepBytes / 16;          // 136 / 72 / 80
    static constexpr int kLoads = (kChunks + 63) / 64;       // 3 / 2 / 2
    static_assert(kStepBytes % 16 == 0, "whole chunks");
    struct Chunks {
        u32x4 v[kLoads];
    };
    // step points at the step's first byte, 16-byte aligned
    __device__ static void fetch(const uint8_t* step, int lane, Chunks& c) {
        const u32x4* p = reinterpret_cast<const u32x4*>(step);
#pragma unroll
        for (int k = 0; k < kLoads; ++k) c.v[k] = __builtin_nontemporal_load(p + min(64 * k + lane, kChunks - 1));
    }
    // The same loads through a buffer descriptor: the step starts soff bytes
    // into the buffer of rs, and voff[k] = 16 * min(64 k + lane, kChunks - 1)
    // (lane_offsets) is the lane's chunk within it.  The address arithmetic
    // is scalar (soff) and per-lane constant (voff), so no vector
    // instructions go to it; offsets past the buffer's range read 0.
    __device__ static void lane_offsets(int lane, int (&voff)[kLoads]) {
#pragma unroll
        for (int k = 0; k < kLoads; ++k) voff[k] = 16 * min(64 * k + lane, kChunks - 1);
    }
    __device__ static void fetch(__amdgpu_buffer_rsrc_t rs, int soff, const int (&voff)[kLoads], Chunks& c) {
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[k], soff, kPolicyNT);
            c.v[k] = u32x4{v[0], v[1], v[2], v[3]};
        }
    }
    // Copies the chunks to the wave's LDS scratch (kStepBytes, 16-byte aligned)
    // and reads block `lane` back.  LDS operations of one wave complete in
    // order, so the next step's copy cannot overtake these reads.
    __device__ static void to_block(const Chunks& c, uint8_t* scratch, int lane, typename F::Raw& r) {
#pragma unroll
        for (int k = 0; k < kLoads; ++k)
            if (64 * k + 64 <= kChunks || 64 * k + lane < kChunks)
                *reinterpret_cast<u32x4*>(scratch + 16 * (64 * k + lane)) = c.v[k];
        F::from_lds(scratch, lane, r);
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
// SiLU(g) = g / (1 + e^-g), in fp32 on the device (expf of the device
// library); g = -inf or +inf give -0 and +inf, NaN stays NaN.
__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

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

// The per-element factors the block dot multiplies with x, in element
// order: Q8_0 the signed codes q; Q4_0 the offset codes times 16, 16 (c - 8);
// Q4_1 the dequantized weights d*c + m (one rounding at most; exact for
// every stored block whose value bits span <= 24).  Term<F> then applies
// the rest of the scale: d, d/16 (exact) or nothing.
//
// Q4_0: a nibble moved to the top half of a byte with its top bit flipped
// reads as the signed byte 16 (c - 8), so one sign-extending convert per
// element gives the offset code, with no sum of x to fold in afterwards.
// Written as shift-then-(xor, and) so that each half is one three-input
// bit operation (plus the shift for the low nibbles): 3 instructions per 8
// codes.
__device__ __forceinline__ void signed_nibbles(uint32_t c, uint32_t& lo, uint32_t& hi) {
    lo = ((c << 4) ^ 0x80808080u) & 0xf0f0f0f0u;   // elements 4i..4i+3
    hi = (c ^ 0x80808080u) & 0xf0f0f0f0u;          // elements 16+4i..16+4i+3
}

// Factors of elements 4i..4i+3 of a block (i = 0..7).
template <class F>
__device__ __forceinline__ void chunk_codes(const uint32_t (&c)[8], int i, float d, float m, float (&q)[4]);
template <>
__device__ __forceinline__ void chunk_codes<Q8_0>(const uint32_t (&c)[8], int i, float, float, float (&q)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = sbyte(c[i], k);
}
template <>
__device__ __forceinline__ void chunk_codes<Q4_0>(const uint32_t (&c)[8], int i, float, float, float (&q)[4]) {
    uint32_t lo, hi;
    signed_nibbles(c[i & 3], lo, hi);
    const uint32_t v = i < 4 ? lo : hi;
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = sbyte(v, k);
}
template <>
__device__ __forceinline__ void chunk_codes<Q4_1>(const uint32_t (&c)[8], int i, float d, float m, float (&q)[4]) {
    const uint32_t v = i < 4 ? (c[i] & 0x0f0f0f0fu) : ((c[i - 4] >> 4) & 0x0f0f0f0fu);
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = __builtin_fmaf(d, ubyte(v, k), m);
}

// All 32 factors of a block (the values chunk_codes gives, in element order).
template <class F>
__device__ __forceinline__ void codes_to_float(const uint32_t (&c)[8], float d, float m, float (&q)[32]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float v[4];
        chunk_codes<F>(c, i, d, m, v);
#pragma unroll
        for (int k = 0; k < 4; ++k) q[4 * i + k] = v[k];
    }
}

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

// s[r][b] = sum_{e<32} factor_r[e] * x_b[e] for R blocks (rows) of the same
// block column and the first w of B columns.  Chunk-outer: each 16-byte
// read of x from LDS serves all R rows, so LDS traffic per weight falls by
// R.  Each s[r][b] accumulates e = 0..31 in order, with the operations of
// dot_cols: the same bits.
template <class F, int R, int B>
__device__ __forceinline__ void dot_multi(const uint32_t (&c)[R][8], const float (&d)[R], const float (&m)[R],
                                          const float* __restrict__ xs, int xstride_b, float (&s)[R][B], int w) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) s[r][b] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float q[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) chunk_codes<F>(c[r], i, d[r], m[r], q[r]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (b < w) {
                const float4 xv = *reinterpret_cast<const float4*>(xs + b * xstride_b + 4 * i);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    s[r][b] = __builtin_fmaf(q[r][0], xv.x, s[r][b]);
                    s[r][b] = __builtin_fmaf(q[r][1], xv.y, s[r][b]);
                    s[r][b] = __builtin_fmaf(q[r][2], xv.z, s[r][b]);
                    s[r][b] = __builtin_fmaf(q[r][3], xv.w, s[r][b]);
                }
            }
        }
    }
}

// Adds a block's term to the running sum, from the block dot s of the
// factors above with x.  Written with explicit operations so that every
// entry point (dense, MoE, any batch width) rounds identically.
template <class F> struct Term;
template <> struct Term<Q8_0> {
    // sum_j d q_j x_j = d * s
    __device__ static float add(float acc, float d, float, float s) { return __builtin_fmaf(d, s, acc); }
};
template <> struct Term<Q4_0> {
    // sum_j d (c_j - 8) x_j = (d / 16) * sum_j 16 (c_j - 8) x_j; d / 16 is exact
    __device__ static float add(float acc, float d, float, float s) { return __builtin_fmaf(d * 0.0625f, s, acc); }
};
template <> struct Term<Q4_1> {
    // sum_j (d c_j + m) x_j = s
    __device__ static float add(float acc, float, float, float s) { return acc + s; }
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
template <int XU, int NT, class XT = float>
struct XStage {
    float4 v[XU];
    __device__ __forceinline__ void load(const XT* __restrict__ x, int K4) {
#pragma unroll
        for (int u = 0; u < XU; ++u) v[u] = XIn<XT>::load4(x + 4 * min((int)threadIdx.x + u * NT, K4 - 1));
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

// Stages the first w of the B activation columns xcol[b][0..32*nb) into
// LDS as xs[b][block][36].  Loads are issued in batches of 4 per thread
// before any is used, so the staging costs a few memory round trips, not
// one per element.  vec: every column is aligned for 4-element loads.
// Ends with a barrier.
template <int B, int NT, class XT = float>
__device__ __forceinline__ void stage_x_cols(const XT* const (&xcol)[B], int nb, float* xs, int w, bool vec) {
    const int K = nb * 32;
    const int tid = threadIdx.x;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        if (b < w) {
            float* dst = xs + b * nb * kXPad;
            if (vec) {
                const XT* src = xcol[b];
                const int K4 = K >> 2;
                auto put = [&](int c, const float4& v) {
                    const int e = 4 * c;
                    *reinterpret_cast<float4*>(dst + (e >> 5) * kXPad + (e & 31)) = v;
                };
                for (int c0 = tid; c0 < K4; c0 += 4 * NT) {
                    const int c1 = c0 + NT, c2 = c0 + 2 * NT, c3 = c0 + 3 * NT;
                    const float4 v0 = XIn<XT>::load4(src + 4 * c0);
                    const float4 v1 = XIn<XT>::load4(src + 4 * min(c1, K4 - 1));
                    const float4 v2 = XIn<XT>::load4(src + 4 * min(c2, K4 - 1));
                    const float4 v3 = XIn<XT>::load4(src + 4 * min(c3, K4 - 1));
                    put(c0, v0);
                    if (c1 < K4) put(c1, v1);
                    if (c2 < K4) put(c2, v2);
                    if (c3 < K4) put(c3, v3);
                }
            } else {
                const XT* src = xcol[b];
                auto put = [&](int e, float v) { dst[(e >> 5) * kXPad + (e & 31)] = v; };
                for (int e0 = tid; e0 < K; e0 += 4 * NT) {
                    const int e1 = e0 + NT, e2 = e0 + 2 * NT, e3 = e0 + 3 * NT;
                    const float v0 = XIn<XT>::load1(src + e0);
                    const float v1 = XIn<XT>::load1(src + min(e1, K - 1));
                    const float v2 = XIn<XT>::load1(src + min(e2, K - 1));
                    const float v3 = XIn<XT>::load1(src + min(e3, K - 1));
                    put(e0, v0);
                    if (e1 < K) put(e1, v1);
                    if (e2 < K) put(e2, v2);
                    if (e3 < K) put(e3, v3);
                }
            }
        }
    }
    __syncthreads();
}

}  // namespace
}  // namespace qmv
