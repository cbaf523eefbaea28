// Q6_K: 256-weight super-blocks of 210 bytes, batch 1..8 matvec and
// dequantization, for gfx950.
//
// Format ("One Native Stack for Private, Continuously-Learning AI", Sec.
// "The Unified Quant Core" lists Q6_K as signed 6-bit, 210 bytes per 256
// weights, without its layout; the layout here is a reading, the
// ggml-compatible one): bytes 0-127 ql (the codes' low 4 bits), 128-191 qh
// (their high 2 bits), 192-207 sc[0..15] (int8, one per 16 weights), 208-209
// d (fp16).  Weight e = 128 h + 32 q + l (h < 2, q < 4, l < 32) has its low
// 4 bits in the low (q < 2) or high (q >= 2) nibble of ql[64 h + 32 (q & 1)
// + l] and its high 2 bits at bits 2q, 2q + 1 of qh[32 h + l];
//   w_e = d sc[e / 16] (c - 32).
//
// Mapping: a lane owns the 64 weights of one half h of a super-block with
// l in [16 lh, 16 lh + 16), all four quarters: 16 bytes of ql for quarters
// 0 and 2, 16 for quarters 1 and 3, 16 of qh, four scales and d.  A
// super-block starts 2 (mod 4) bytes into W on every other index, so each
// 16-byte piece is read as 4-byte-aligned words and re-aligned with
// v_alignbyte; every load stays inside the matrix.  A code is rebuilt in
// place as the signed byte 4 (c - 32) (its 4 low bits moved to bits 2-5,
// its 2 high bits to bits 6-7 with the top bit flipped), so one
// sign-extending convert per weight gives it; each 16-weight sum is scaled
// by d sc / 4 (exact: 11 + 8 significant bits) and no offset is folded out
// of a sum.  Activations are staged in LDS as fp32 in the lanes' order (68
// floats per lane's 64 weights: conflict-free 16-byte reads).  Segments of
// LPR lanes reduce in a fixed order: deterministic, and a column's sums are
// the same at every batch width.
#include "qmv_superblock.h"

namespace qmv {
namespace {

constexpr int kQ6KBytes = 210;    // per super-block

// The stored bytes a lane needs for one step, as loaded (4-byte aligned
// words; sh = 2 when the super-block starts 2 bytes past a word).
struct Q6KRaw {
    u32x4 a; uint32_t a4;   // ql bytes 64h + 16lh .. +16 (quarters 0, 2)
    u32x4 b; uint32_t b4;   // ql bytes 64h + 32 + 16lh .. +16 (quarters 1, 3)
    u32x4 c; uint32_t c4;   // qh bytes 32h + 16lh .. +16
    u32x4 t; uint32_t u;    // scales sc[0..15] (and 2 bytes before when sh = 2), sc[14..15]
    uint32_t dh;            // d (fp16 bits)
    uint32_t sh;            // 0, or 2 when the super-block starts 2 bytes past a word
};

__device__ __forceinline__ void q6k_fetch(const uint8_t* sb, int hl, Q6KRaw& r) {
    const int sh = (int)(reinterpret_cast<uintptr_t>(sb) & 2);
    const uint8_t* p = sb - sh;                       // 4-byte aligned
    const int pa = 64 * (hl >> 1) + 16 * (hl & 1);
    const int pc = 128 + 32 * (hl >> 1) + 16 * (hl & 1);
    r.a = ld16(p + pa);
    r.a4 = ld4(p + pa + 16);
    r.b = ld16(p + pa + 32);
    r.b4 = ld4(p + pa + 48);
    r.c = ld16(p + pc);
    r.c4 = ld4(p + pc + 16);
    r.t = ld16(p + 192);
    r.u = ld2(sb + 206);
    r.dh = ld2(sb + 208);
    r.sh = (uint32_t)sh;
}

// Rebuilds the lane's 16-byte pieces at their true alignment.
__device__ __forceinline__ void realign(const u32x4& v, uint32_t e, uint32_t sh, uint32_t (&o)[4]) {
    const uint32_t w[5] = {v.x, v.y, v.z, v.w, e};
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
}

// Four codes of quarter q as signed bytes 4 (c - 32): lo holds their 4 low
// bits at bits 0-3 (q < 2) or 4-7 (q >= 2) of each byte, hf the qh word
// with the top bit of every 2-bit field flipped.  4 operations per word for
// a constant q, 6 for a run-time one.
__device__ __forceinline__ uint32_t q6k_bytes(uint32_t lo, uint32_t hf, int q) {
    const uint32_t l = q < 2 ? (lo << 2) : (lo >> 2);          // low bits to bits 2-5
    const uint32_t h = (hf << (6 - 2 * q)) & 0xc0c0c0c0u;     // field q to bits 6-7
    return (l & 0x3c3c3c3cu) | h;
}

// Staged activations: the 64 x values of lane group g = 4 sb + 2 h + lh
// (elements 256 sb + 128 h + 32 q + 16 lh + i) at xs[g * kSbXPad + 16 q +
// i], so a lane reads its quarter's 16 values contiguously and lanes on
// consecutive groups start 4 banks apart.
__device__ __forceinline__ int q6k_slot(int e) {
    const int g = ((e >> 8) << 2) | (((e >> 7) & 1) << 1) | ((e >> 4) & 1);
    return g * kSbXPad + 16 * ((e >> 5) & 3) + (e & 15);
}

// A wave step covers RW = 64 / LPR rows, one per segment of LPR lanes; lane
// li of a segment takes lane group li + LPR t of its row in step t.
template <int B, int LPR, int NW, class XT, bool ROUTE>
__global__ __launch_bounds__(64 * NW) void q6k_kernel(const uint8_t* __restrict__ W, int64_t N, int nsb,
                                                       const XT* __restrict__ x, int64_t ldx, float* __restrict__ y,
                                                       int64_t ldy, int xvec, const SbRoute route) {
    bool bad = false;   // routed pair with an invalid expert id: its outputs become NaN
    if constexpr (ROUTE) bad = sb_route(route, W, x, y, ldy);
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* xs = lds;                          // [B][4 nsb][kSbXPad], in q6k_slot order
    constexpr int RW = 64 / LPR;              // rows per tile
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int G = 4 * nsb;                    // lane groups (64 weights) per row
    const int T = (G + LPR - 1) / LPR;        // steps per row
    const int64_t pitch = (int64_t)nsb * kQ6KBytes;
    const int64_t ntiles = (N + RW - 1) / RW;
    const int64_t wstride = (int64_t)gridDim.x * NW;

    auto load_step = [&](int64_t tile, int t, Q6KRaw& r) {
        const int g = min(li + LPR * t, G - 1);                 // clamp: stays in bounds
        const int64_t row = min(tile * RW + seg, N - 1);
        q6k_fetch(W + row * pitch + (int64_t)(g >> 2) * kQ6KBytes, g & 3, r);
    };

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
    auto compute_step = [&](int64_t tile, int t, const Q6KRaw& r) {
        const int g = li + LPR * t;
        const bool valid = g < G;
        const int gc = valid ? g : G - 1;
        const bool h = (gc & 2) != 0;          // half of the super-block
        const int lh = gc & 1;                 // l in [16 lh, 16 lh + 16)
        uint32_t A[4], Bq[4], C[4], S[4];
        realign(r.a, r.a4, r.sh, A);
        realign(r.b, r.b4, r.sh, Bq);
        realign(r.c, r.c4, r.sh, C);
        realign(r.t, r.u, r.sh, S);
        // the lane's quarter q uses sc[8 h + 2 q + lh]; d sc / 4 is exact
        const float d4 = half_bits_to_float(r.dh) * 0.25f;
        const uint32_t s01 = h ? S[2] : S[0], s23 = h ? S[3] : S[1];
        uint32_t hf[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) hf[k] = C[k] ^ 0xaaaaaaaau;   // top bit of each 2-bit field flipped
        const float* xg = xs + gc * kSbXPad;
        const int cs = G * kSbXPad;            // column stride in LDS
        float st[B];
#pragma unroll
        for (int b = 0; b < B; ++b) st[b] = 0.f;
        // quarter q: 16 weights, one scale; st += (d sc / 4) * sum 4 (c - 32) x
        auto quarter = [&](int q) {
            const float scale = d4 * (float)(int8_t)((q < 2 ? s01 : s23) >> (8 * lh + 16 * (q & 1)));
            float s[B];
#pragma unroll
            for (int b = 0; b < B; ++b) s[b] = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t v = q6k_bytes((q & 1) ? Bq[k] : A[k], hf[k], q);
                const float c0 = sbyte(v, 0), c1 = sbyte(v, 1), c2 = sbyte(v, 2), c3 = sbyte(v, 3);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float4 xv = *reinterpret_cast<const float4*>(xg + b * cs + 16 * q + 4 * k);
                    s[b] = __builtin_fmaf(c0, xv.x, s[b]);
                    s[b] = __builtin_fmaf(c1, xv.y, s[b]);
                    s[b] = __builtin_fmaf(c2, xv.z, s[b]);
                    s[b] = __builtin_fmaf(c3, xv.w, s[b]);
                }
            }
#pragma unroll
            for (int b = 0; b < B; ++b) st[b] = __builtin_fmaf(scale, s[b], st[b]);
        };
        // One column: the quarters unrolled (constant shifts and selects).
        // More columns: a loop that is not unrolled, so the quarters share
        // registers (unrolled, the scheduler interleaves them: 180 VGPRs at
        // batch 2, spills from batch 4).
        if constexpr (B == 1) {
#pragma unroll
            for (int q = 0; q < 4; ++q) quarter(q);
        } else {
#pragma unroll 1
            for (int q = 0; q < 4; ++q) quarter(q);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = valid ? acc[b] + st[b] : acc[b];
        if (t == T - 1) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float tot = segment_sum<LPR>(acc[b]);
                const int64_t row = tile * RW + seg;
                if (li == 0 && row < N) y[b * ldy + row] = bad ? __builtin_nanf("") : tot;
                acc[b] = 0.f;
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
    Q6KRaw buf[2];
    auto load_next = [&](Q6KRaw& r) {
        load_step(min(ltile, ntiles - 1), ltile < ntiles ? lt : 0, r);
        if (ltile < ntiles) advance(ltile, lt);
    };
    // the first weight loads go out before the staging
    load_next(buf[0]);
    {
        const XT* xcol[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xcol[b] = x + b * ldx;
        sb_stage_x<B, 64 * NW, XT>(xcol, kSbWeights * nsb, xs, xvec != 0, q6k_slot);   // ends with a barrier
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

// One lane group's sum (64 weights) for one column, in q6k_kernel's order
// at batch 1 (quarters 0..3, each 16-weight sum scaled by d sc / 4 into a
// running fma): bitwise that kernel's step sum.
__device__ __forceinline__ float q6k_group_sum(const Q6KRaw& r, int gc, const float* xg) {
    const bool h = (gc & 2) != 0;
    const int lh = gc & 1;
    uint32_t A[4], Bq[4], C[4], S[4];
    realign(r.a, r.a4, r.sh, A);
    realign(r.b, r.b4, r.sh, Bq);
    realign(r.c, r.c4, r.sh, C);
    realign(r.t, r.u, r.sh, S);
    const float d4 = half_bits_to_float(r.dh) * 0.25f;
    const uint32_t s01 = h ? S[2] : S[0], s23 = h ? S[3] : S[1];
    uint32_t hf[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) hf[k] = C[k] ^ 0xaaaaaaaau;
    float st = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float scale = d4 * (float)(int8_t)((q < 2 ? s01 : s23) >> (8 * lh + 16 * (q & 1)));
        float sq = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = q6k_bytes((q & 1) ? Bq[k] : A[k], hf[k], q);
            const float4 xv = *reinterpret_cast<const float4*>(xg + 16 * q + 4 * k);
            sq = __builtin_fmaf(sbyte(v, 0), xv.x, sq);
            sq = __builtin_fmaf(sbyte(v, 1), xv.y, sq);
            sq = __builtin_fmaf(sbyte(v, 2), xv.z, sq);
            sq = __builtin_fmaf(sbyte(v, 3), xv.w, sq);
        }
        st = __builtin_fmaf(scale, sq, st);
    }
    return st;
}

// The Q6_K step for the kernels over a format's step (sb_group_kernel,
// sb_combine_kernel, sb_swiglu_kernel): a lane's 64 weights and their
// batch-1 sum.
struct Q6KOps {
    using Raw = Q6KRaw;
    static constexpr int kBytes = kQ6KBytes;
    static constexpr int kWaves = 1;          // the compiler's choice
    __device__ static void fetch(const uint8_t* row, int g, Raw& r) {
        q6k_fetch(row + (int64_t)(g >> 2) * kQ6KBytes, g & 3, r);
    }
    __device__ static float group_sum(const Raw& r, int, int gc, const float* xs) {
        return q6k_group_sum(r, gc, xs + gc * kSbXPad);
    }
    __device__ static int slot(int e) { return q6k_slot(e); }
};

// One thread per 16-weight sub-block: out = (d sc / 4) * 4 (c - 32), the
// weight the matvec uses (exact).
__global__ __launch_bounds__(kThreads) void q6k_dequant_kernel(const uint8_t* __restrict__ W, int64_t nsub,
                                                               float* __restrict__ out) {
    const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (u >= nsub) return;
    const uint8_t* sb = W + (u >> 4) * kQ6KBytes;
    const int s = (int)(u & 15);               // sub-block: weights 16 s .. 16 s + 15
    const int h = s >> 3, q = (s >> 1) & 3, lh = s & 1;
    const float scale = half_bits_to_float(sb[208] | (sb[209] << 8)) * 0.25f * (float)(int8_t)sb[192 + s];
    const uint8_t* ql = sb + 64 * h + 32 * (q & 1) + 16 * lh;
    const uint8_t* qh = sb + 128 + 32 * h + 16 * lh;
    float* o = out + u * 16;
    for (int i = 0; i < 16; ++i) {
        const int lo = q < 2 ? (ql[i] & 15) : (ql[i] >> 4);
        const int c = lo | (((qh[i] >> (2 * q)) & 3) << 4);
        o[i] = scale * (float)(4 * (c - 32));
    }
}

struct Q6KFormat {
    static constexpr qmv_fmt kFmt = QMV_Q6_K;
    static constexpr const char* kLabel = "Q6_K";
    static constexpr const char* kEntry = "qmv_q6_k";
    static constexpr int kWAlign = 4;          // 4-byte-aligned loads, re-aligned in registers
    static constexpr bool kMfma = true;        // batch 2..8: q6k_mma_kernel
    static constexpr bool kSwiglu = true;      // MoE gate||up with SiLU(gate) * up fused (sb_swiglu_kernel)
    static constexpr bool kCombine = true;     // MoE down with the weighted combine fused
    template <int LPR, int NW>
    static auto combine_kernel() { return sb_combine_kernel<Q6KOps, LPR, NW>; }
    static constexpr bool kGroup = true;       // qmv_chain: shared-input stages as one launch
    template <int LPR, int NW>
    static auto group_kernel() { return sb_group_kernel<Q6KOps, LPR, NW>; }
    template <int LPR, int NW, class XT>
    static auto swiglu_kernel() { return sb_swiglu_kernel<Q6KOps, LPR, NW, XT>; }
    static constexpr int kDequantWeights = 16;
    static constexpr int kBytes = kQ6KBytes;
    template <int B, int LPR, int NW, class XT, bool ROUTE, bool SW = false>
    static auto kernel() { return q6k_kernel<B, LPR, NW, XT, ROUTE>; }
    static auto dequant_kernel() { return q6k_dequant_kernel; }
};

}  // namespace

const FormatOps& ops_q6_k() { return sb_format_ops<Q6KFormat>(); }

}  // namespace qmv

extern "C" int32_t qmv_q6_k(const void* W, int64_t n_rows, int64_t n_cols, const float* x, int64_t ldx, int32_t batch,
                            float* y, int64_t ldy, void* stream) {
    return qmv::ops_q6_k().matvec("qmv_q6_k", W, n_rows, n_cols, x, QMV_X_F32, ldx, batch, y, ldy, stream,
                                  QMV_PATH_AUTO);
}
