// Q4_K: 256-weight super-blocks of 144 bytes, batch 1..8 matvec and
// dequantization, for gfx950.
//
// Format ("One Native Stack for Private, Continuously-Learning AI", Sec.
// "The Unified Quant Core" names Q4_K among the formats of the one quant
// core but gives no layout; the layout here is a reading, the
// ggml-compatible one): bytes 0-1 d (fp16), 2-3 dmin (fp16), 4-15 b[0..11]
// holding eight 6-bit sub-block scales sc_s and minimums mn_s
//   s < 4:  sc_s = b[s] & 63,                     mn_s = b[s+4] & 63
//   s >= 4: sc_s = (b[s+4] & 15) + 16 (b[s-4] >> 6), mn_s = (b[s+4] >> 4) + 16 (b[s] >> 6)
// and 16-143 q[0..127]: weight 32 s + i is the low nibble of
// q[32 (s/2) + i] for even s, the high nibble for odd s;
//   w = d sc_s c - dmin mn_s.
//
// Mapping: a lane owns one 64-weight group (sub-blocks 2p and 2p + 1 of a
// super-block, which share 32 code bytes): per step it loads the 16-byte
// super-block header and its 32 code bytes with three aligned 16-byte loads
// (the four lanes of a super-block read the same header line).  Each weight
// is dequantized on its own, w = fma(d sc, c, -dmin mn) with d sc and
// dmin mn exact in fp32, so a w is the exact value rounded once and no
// offset is folded out of a sum (rows of mostly zero weights keep the
// per-output bound).  Activations are staged in LDS as fp32 (16-bit inputs
// widened exactly).  Segments of LPR lanes reduce in a fixed order, so the
// result is deterministic and a column's sums are the same at every batch
// width.
#include "qmv_superblock.h"

namespace qmv {
namespace {

constexpr int kQ4KBytes = 144;    // per super-block

struct Q4KGroup {
    u32x4 h;        // d, dmin, b[0..11]
    u32x4 c0, c1;   // the group's 32 code bytes
};

__device__ __forceinline__ u32x4 ld16_aligned(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// The 32 codes of one Q4_K sub-block as a dot_multi format: element 4 i + k
// is byte k of c[i], the code already isolated in its byte (as c, or as
// 16 c in the high half); the factor is fma(d, byte, m), the weight itself,
// with d = d sc (or d sc / 16) and m = -dmin mn.
struct Q4KSub {};
template <>
__device__ __forceinline__ void chunk_codes<Q4KSub>(const uint32_t (&c)[8], int i, float d, float m, float (&q)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = __builtin_fmaf(d, ubyte(c[i], k), m);
}

// The 6-bit scale and minimum of sub-block s (0..7); h.y, h.z, h.w hold
// b[0..3], b[4..7], b[8..11] (byte k of a word at bits 8k).
__device__ __forceinline__ void q4k_scale_min(const u32x4& h, int s, int& sc, int& mn) {
    const int t = 8 * (s & 3);
    const uint32_t y = h.y >> t, z = h.z >> t, w = h.w >> t;
    const int sc_lo = (int)(y & 63), mn_lo = (int)(z & 63);
    const int sc_hi = (int)((w & 15) | (((y >> 6) & 3) << 4));
    const int mn_hi = (int)(((w >> 4) & 15) | (((z >> 6) & 3) << 4));
    sc = s < 4 ? sc_lo : sc_hi;
    mn = s < 4 ? mn_lo : mn_hi;
}

// The scales and minimums of sub-blocks 2 part and 2 part + 1 together:
// the two sub-blocks' bytes are spread into the low bytes of a word's two
// 16-bit halves, so one shift and mask decode both.  The selectors and the
// mask depend only on part, which is fixed per lane (a lane's groups are
// li + LPR t with LPR a multiple of 4).  For part < 2 the fields are the
// low six bits of b[s] (scale) and b[s+4] (minimum); for part >= 2 the low
// four bits come from b[s+4] (scale: its low nibble, minimum: its high
// nibble) and the top two from bits 6, 7 of b[s-4] and b[s].
struct Q4KPairSel {
    uint32_t sel;    // bytes o, o+1 of the first operand (part >= 2) or of the second
    uint32_t selp;   // bytes o, o+1 of the second operand (part >= 2), else zeros
    uint32_t ma;     // mask of the low field: 6 bits (part < 2) or 4
};
__device__ __forceinline__ Q4KPairSel q4k_pair_sel(int part) {
    const uint32_t o = 2 * (part & 1);
    const bool hi = part >= 2;
    const uint32_t b0 = (hi ? 4u : 0u) + o;
    Q4KPairSel ps;
    ps.sel = b0 | (0x0cu << 8) | ((b0 + 1) << 16) | (0x0cu << 24);   // 0x0c selects a zero byte
    ps.selp = hi ? (o | (0x0cu << 8) | ((o + 1) << 16) | (0x0cu << 24)) : 0x0c0c0c0cu;
    ps.ma = hi ? 0x000f000fu : 0x003f003fu;
    return ps;
}
// sc2, mn2: the scales and minimums of the two sub-blocks in bytes 0 and 2.
__device__ __forceinline__ void q4k_pair_scales(const u32x4& h, const Q4KPairSel& ps, uint32_t& sc2, uint32_t& mn2) {
    // h.y = b[0..3], h.z = b[4..7], h.w = b[8..11]; byte k of h.w >> 4
    // holds the high nibble of b[8+k] in its low four bits
    const uint32_t a_sc = __builtin_amdgcn_perm(h.w, h.y, ps.sel);
    const uint32_t a_mn = __builtin_amdgcn_perm(h.w >> 4, h.z, ps.sel);
    const uint32_t yp = __builtin_amdgcn_perm(0u, h.y, ps.selp);
    const uint32_t zp = __builtin_amdgcn_perm(0u, h.z, ps.selp);
    sc2 = (a_sc & ps.ma) | ((yp >> 2) & 0x00300030u);
    mn2 = (a_mn & ps.ma) | ((zp >> 2) & 0x00300030u);
}

// A wave step covers RW = 64 / LPR rows, one per segment of LPR lanes.
// (Two rows per lane, each staged activation read feeding both, measured
// slower at every batch width: 123-228 VGPRs against 63-160.)  SW (routed,
// one column): every expert holds 2N rows, gate rows then up rows, and the
// segment of output row i streams gate row i and up row N + i in the same
// lanes and steps (two rows per lane, each row's sums as in the one-row
// form), then writes SiLU(gate) * up.
template <int B, int LPR, int NW, class XT, bool ROUTE, bool SW = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(B == 1 && !SW ? 8 : 1))) void q4k_kernel(
    const uint8_t* __restrict__ W, int64_t N, int nsb, const XT* __restrict__ x, int64_t ldx, float* __restrict__ y,
    int64_t ldy, int xvec, const SbRoute route) {
    static_assert(!SW || (ROUTE && B == 1), "the fused SwiGLU form is routed, one column");
    constexpr int NR = SW ? 2 : 1;            // rows per lane
    bool bad = false;   // routed pair with an invalid expert id: its outputs become NaN
    if constexpr (ROUTE) bad = sb_route(route, W, x, y, ldy);
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* xs = lds;                          // [B][4 nsb][kSbXPad], x[b][64 g + e] at [b][g][e]
    constexpr int RW = 64 / LPR;              // rows per tile
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int G = 4 * nsb;                    // 64-weight groups per row
    const int T = (G + LPR - 1) / LPR;        // steps per row
    const int64_t pitch = (int64_t)nsb * kQ4KBytes;
    const int64_t ntiles = (N + RW - 1) / RW;
    const int64_t wstride = (int64_t)gridDim.x * NW;

    // A step's loads: the tile's first row as a wave-uniform base and 32-bit
    // lane offsets from it (a tile spans RW rows of at most 150 super-blocks).
    struct Step {
        Q4KGroup r[NR];                       // [1]: the up row N + i (SW)
    };
    auto load_step = [&](int64_t tile, int t, Step& st) {
        const int g = min(li + LPR * t, G - 1);                 // clamp: stays in bounds
        const int64_t r0 = tile * RW;                            // tile < ntiles: r0 < N
        const int64_t rem = N - 1 - r0;
        const int lim = __builtin_amdgcn_readfirstlane(rem < RW - 1 ? (int)rem : RW - 1);
        const int lr = min(seg, lim);                            // rows past the end: the last row
        const uint32_t off = __umul24((uint32_t)lr, (uint32_t)pitch) + (uint32_t)(g >> 2) * kQ4KBytes;
        const uint32_t coff = off + 16 + 32 * (g & 3);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const uint8_t* base = W + (r0 + k * N) * pitch;
            st.r[k].h = ld16_aligned(base + off);
            st.r[k].c0 = ld16_aligned(base + coff);
            st.r[k].c1 = ld16_aligned(base + coff + 16);
        }
    };

    float acc[NR][B];
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[k][b] = 0.f;
    // part = g & 3 for every group g of the lane (on a clamped step past the
    // row's end the result is discarded)
    const Q4KPairSel ps = q4k_pair_sel(li & 3);
    auto compute_step = [&](int64_t tile, int t, const Step& st) {
        const int g = li + LPR * t;
        const bool valid = g < G;
        const int gc = valid ? g : G - 1;
        float da[NR], ma[NR], db16[NR], mb[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const u32x4& h = st.r[k].h;
            const float d = half_bits_to_float(h.x);
            const float dmin = half_bits_to_float(h.x >> 16);
            uint32_t sc2, mn2;
            q4k_pair_scales(h, ps, sc2, mn2);
            // exact: 11 + 6 significant bits each (and d sc / 16 exact too)
            da[k] = d * ubyte(sc2, 0);
            ma[k] = dmin * ubyte(mn2, 0);
            db16[k] = (d * 0.0625f) * ubyte(sc2, 2);
            mb[k] = dmin * ubyte(mn2, 2);
        }
        // Sub-block 2 part (the low nibbles of the 32 code bytes), then
        // 2 part + 1 (the high nibbles): a loop that is not unrolled, so the
        // two halves share registers.
        float s[NR][B];
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int b = 0; b < B; ++b) s[k][b] = 0.f;
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            // low nibbles as c; high nibbles in place, as 16 c, with the
            // scale d sc / 16 (exact): the same products either way
            const uint32_t mask = h ? 0xf0f0f0f0u : 0x0f0f0f0fu;
            uint32_t c[NR][8];
            float fd[NR], fm[NR];
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                const Q4KGroup& r = st.r[k];
                const uint32_t w8[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) c[k][i] = opaque_bits(w8[i] & mask);
                fd[k] = h ? db16[k] : da[k];
                fm[k] = h ? -mb[k] : -ma[k];
            }
            float sh_dot[NR][B];
            dot_multi<Q4KSub, NR, B>(c, fd, fm, xs + gc * kSbXPad + 32 * h, G * kSbXPad, sh_dot, B);
#pragma unroll
            for (int k = 0; k < NR; ++k)
#pragma unroll
                for (int b = 0; b < B; ++b) s[k][b] += sh_dot[k][b];
        }
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[k][b] = valid ? acc[k][b] + s[k][b] : acc[k][b];
        if (t == T - 1) {
            const int64_t row = tile * RW + seg;
            if constexpr (SW) {
                const float gs = segment_sum<LPR>(acc[0][0]);
                const float us = segment_sum<LPR>(acc[1][0]);
                if (li == 0 && row < N) y[row] = bad ? __builtin_nanf("") : silu(gs) * us;
                acc[0][0] = acc[1][0] = 0.f;
            } else {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float tot = segment_sum<LPR>(acc[0][b]);
                    if (li == 0 && row < N) y[b * ldy + row] = bad ? __builtin_nanf("") : tot;
                    acc[0][b] = 0.f;
                }
            }
        }
    };
    auto advance = [&](int64_t& tile, int& t) {
        if (++t == T) {
            t = 0;
            tile += wstride;
        }
    };

    int64_t ltile = (int64_t)blockIdx.x * NW + wave;   // next step to load
    int lt = 0;
    int64_t ctile = ltile;                             // next step to compute
    int ct = 0;
    Step buf[2];
    auto load_next = [&](Step& r) {
        load_step(min(ltile, ntiles - 1), ltile < ntiles ? lt : 0, r);
        if (ltile < ntiles) advance(ltile, lt);
    };
    // the first weight loads go out before the staging
    load_next(buf[0]);
    {
        const XT* xcol[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xcol[b] = x + b * ldx;
        // groups of 64 in order, each padded to kSbXPad floats; ends with a barrier
        sb_stage_x<B, 64 * NW, XT>(xcol, kSbWeights * nsb, xs, xvec != 0,
                                   [](int e) { return (e >> 6) * kSbXPad + (e & 63); });
    }
    // Two register buffers used in turn; once the load cursor is past the
    // wave's last step, the step in hand is the last one: it is computed
    // after the loop and nothing more is loaded.
    if (ctile < ntiles) {
        while (ltile < ntiles) {
            load_next(buf[1]);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(ctile, ct, buf[0]);
            advance(ctile, ct);
            if (ltile >= ntiles) {
                buf[0] = buf[1];
                break;
            }
            load_next(buf[0]);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(ctile, ct, buf[1]);
            advance(ctile, ct);
        }
        compute_step(ctile, ct, buf[0]);
    }
}

// One 64-weight group's sum for one column, in q4k_kernel's order (the two
// halves in turn through dot_multi): bitwise that kernel's step sum.
__device__ __forceinline__ float q4k_group_sum(const Q4KGroup& r, const Q4KPairSel& ps, const float* xg) {
    const float d = half_bits_to_float(r.h.x);
    const float dmin = half_bits_to_float(r.h.x >> 16);
    uint32_t sc2, mn2;
    q4k_pair_scales(r.h, ps, sc2, mn2);
    const float da = d * ubyte(sc2, 0), ma = dmin * ubyte(mn2, 0);
    const float db16 = (d * 0.0625f) * ubyte(sc2, 2), mb = dmin * ubyte(mn2, 2);
    float s = 0.f;
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
        const uint32_t mask = h ? 0xf0f0f0f0u : 0x0f0f0f0fu;
        const uint32_t w8[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
        uint32_t c[1][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c[0][i] = opaque_bits(w8[i] & mask);
        const float fd[1] = {h ? db16 : da}, fm[1] = {h ? -mb : -ma};
        float sh[1][1];
        dot_multi<Q4KSub, 1, 1>(c, fd, fm, xg + 32 * h, 0, sh, 1);
        s += sh[0][0];
    }
    return s;
}

// The Q4_K step for the kernels over a format's step (sb_group_kernel,
// sb_combine_kernel): a lane's group of 64 weights and its batch-1 sum.
struct Q4KOps {
    using Raw = Q4KGroup;
    static constexpr int kBytes = kQ4KBytes;
    static constexpr int kWaves = 5;          // 71-89 VGPRs, no spills
    __device__ static void fetch(const uint8_t* row, int g, Raw& r) {
        const uint8_t* sb = row + (int64_t)(g >> 2) * kQ4KBytes;
        const int coff = 16 + 32 * (g & 3);
        r.h = ld16_aligned(sb);
        r.c0 = ld16_aligned(sb + coff);
        r.c1 = ld16_aligned(sb + coff + 16);
    }
    __device__ static float group_sum(const Raw& r, int li, int gc, const float* xs) {
        return q4k_group_sum(r, q4k_pair_sel(li & 3), xs + gc * kSbXPad);
    }
    __device__ static int slot(int e) { return (e >> 6) * kSbXPad + (e & 63); }
};

// One thread per 32-weight sub-block: out = fma(d sc, c, -dmin mn), the
// same value the matvec uses for each weight.
__global__ __launch_bounds__(kThreads) void q4k_dequant_kernel(const uint8_t* __restrict__ W, int64_t nsub,
                                                               float* __restrict__ out) {
    const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (u >= nsub) return;
    const int64_t sbi = u >> 3;
    const int s = (int)(u & 7);
    const uint8_t* sb = W + sbi * kQ4KBytes;
    const u32x4 h = ld16_aligned(sb);
    int sc, mn;
    q4k_scale_min(h, s, sc, mn);
    const float ds = half_bits_to_float(h.x) * (float)sc;
    const float dm = half_bits_to_float(h.x >> 16) * (float)mn;
    const uint8_t* q = sb + 16 + 32 * (s >> 1);
    float* o = out + u * 32;
    for (int i = 0; i < 32; ++i) {
        const int c = (s & 1) ? (q[i] >> 4) : (q[i] & 15);
        o[i] = __builtin_fmaf(ds, (float)c, -dm);
    }
}

struct Q4KFormat {
    static constexpr qmv_fmt kFmt = QMV_Q4_K;
    static constexpr const char* kLabel = "Q4_K";
    static constexpr const char* kEntry = "qmv_q4_k";
    static constexpr int kWAlign = 16;         // the kernel's aligned 16-byte loads
    static constexpr bool kMfma = true;        // batch 2..8: Mma<Q4KSuper> in the matrix-core kernel
    static constexpr bool kSwiglu = true;      // MoE gate||up with SiLU(gate) * up fused (routed kernel)
    static constexpr bool kCombine = true;     // MoE down with the weighted combine fused
    template <int LPR, int NW>
    static auto combine_kernel() { return sb_combine_kernel<Q4KOps, LPR, NW>; }
    static constexpr bool kGroup = true;       // qmv_chain: shared-input stages as one launch
    template <int LPR, int NW>
    static auto group_kernel() { return sb_group_kernel<Q4KOps, LPR, NW>; }
    template <int LPR, int NW, class XT>
    static auto swiglu_kernel() { return q4k_kernel<1, LPR, NW, XT, true, true>; }
    static constexpr int kDequantWeights = 32;
    static constexpr int kBytes = kQ4KBytes;
    template <int B, int LPR, int NW, class XT, bool ROUTE, bool SW = false>
    static auto kernel() { return q4k_kernel<B, LPR, NW, XT, ROUTE, SW>; }
    static auto dequant_kernel() { return q4k_dequant_kernel; }
};

}  // namespace

const FormatOps& ops_q4_k() { return sb_format_ops<Q4KFormat>(); }

}  // namespace qmv

extern "C" int32_t qmv_q4_k(const void* W, int64_t n_rows, int64_t n_cols, const float* x, int64_t ldx, int32_t batch,
                            float* y, int64_t ldy, void* stream) {
    return qmv::ops_q4_k().matvec("qmv_q4_k", W, n_rows, n_cols, x, QMV_X_F32, ldx, batch, y, ldy, stream,
                                  QMV_PATH_AUTO);
}
