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
#include <algorithm>

#include "qmv_block_decode.h"

namespace qmv {
namespace {

constexpr int kQ4KBytes = 144;    // per super-block
constexpr int kQ4KWeights = 256;

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

// Staged activations: x[b][64 g + e] at xs[b][g][e] with groups padded to
// 68 floats, so the 16-byte reads of lanes on consecutive groups start 4
// banks apart and a wave's read is free of bank conflicts (with 32-weight
// blocks of 36 floats, lanes two blocks apart would collide two ways).
constexpr int kQ4KXPad = 68;

// Stages w of the B columns xcol[b][0..K) into LDS in that layout; loads in
// batches of 4 per thread before any is stored.  vec: every column aligned
// for 4-element loads.  Ends with a barrier.
template <int B, int NT, class XT>
__device__ __forceinline__ void q4k_stage_x(const XT* const (&xcol)[B], int K, float* xs, bool vec) {
    const int G = K >> 6;
    const int tid = threadIdx.x;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float* dst = xs + b * G * kQ4KXPad;
        const XT* src = xcol[b];
        if (vec) {
            const int K4 = K >> 2;
            auto put = [&](int c, const float4& v) {
                const int e = 4 * c;
                *reinterpret_cast<float4*>(dst + (e >> 6) * kQ4KXPad + (e & 63)) = v;
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
            auto put = [&](int e, float v) { dst[(e >> 6) * kQ4KXPad + (e & 63)] = v; };
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
    __syncthreads();
}

// Hides a value's bits from the optimizer: a masked word then converts with
// one byte-select convert per element instead of a bit-field extract and a
// convert.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
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

// A wave step covers RW = 64 / LPR rows, one per segment of LPR lanes.
// (Two rows per lane, each staged activation read feeding both, measured
// slower at every batch width: 123-228 VGPRs against 63-160.)
template <int B, int LPR, int NW, class XT>
__global__ __launch_bounds__(64 * NW) void q4k_kernel(const uint8_t* __restrict__ W, int64_t N, int nsb,
                                                       const XT* __restrict__ x, int64_t ldx, float* __restrict__ y,
                                                       int64_t ldy, int xvec) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* xs = lds;                          // [B][4 nsb][kQ4KXPad]
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

    auto load_step = [&](int64_t tile, int t, Q4KGroup& r) {
        const int g = min(li + LPR * t, G - 1);                 // clamp: stays in bounds
        const int64_t row = min(tile * RW + seg, N - 1);
        const uint8_t* sb = W + row * pitch + (int64_t)(g >> 2) * kQ4KBytes;
        const int coff = 16 + 32 * (g & 3);
        r.h = ld16_aligned(sb);
        r.c0 = ld16_aligned(sb + coff);
        r.c1 = ld16_aligned(sb + coff + 16);
    };

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
    auto compute_step = [&](int64_t tile, int t, const Q4KGroup& r) {
        const int g = li + LPR * t;
        const bool valid = g < G;
        const int gc = valid ? g : G - 1;
        const int part = gc & 3;
        const float d = half_bits_to_float(r.h.x);
        const float dmin = half_bits_to_float(r.h.x >> 16);
        int sca, mna, scb, mnb;
        q4k_scale_min(r.h, 2 * part, sca, mna);
        q4k_scale_min(r.h, 2 * part + 1, scb, mnb);
        // exact: 11 + 6 significant bits each
        const float da = d * (float)sca, ma = dmin * (float)mna;
        const float db = d * (float)scb, mb = dmin * (float)mnb;
        // Sub-block 2 part (the low nibbles of the 32 code bytes), then
        // 2 part + 1 (the high nibbles): a loop that is not unrolled, so the
        // two halves share registers.
        float s[B];
#pragma unroll
        for (int b = 0; b < B; ++b) s[b] = 0.f;
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            // low nibbles as c; high nibbles in place, as 16 c, with the
            // scale d sc / 16 (exact): the same products either way
            const uint32_t mask = h ? 0xf0f0f0f0u : 0x0f0f0f0fu;
            const uint32_t w8[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
            uint32_t c[1][8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[0][i] = opaque(w8[i] & mask);
            const float fd[1] = {h ? db * 0.0625f : da}, fm[1] = {h ? -mb : -ma};
            float sh_dot[1][B];
            dot_multi<Q4KSub, 1, B>(c, fd, fm, xs + gc * kQ4KXPad + 32 * h, G * kQ4KXPad, sh_dot, B);
#pragma unroll
            for (int b = 0; b < B; ++b) s[b] += sh_dot[0][b];
        }
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = valid ? acc[b] + s[b] : acc[b];
        if (t == T - 1) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float tot = segment_sum<LPR>(acc[b]);
                const int64_t row = tile * RW + seg;
                if (li == 0 && row < N) y[b * ldy + row] = tot;
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
    Q4KGroup buf[2];
    auto load_next = [&](Q4KGroup& r) {
        load_step(min(ltile, ntiles - 1), ltile < ntiles ? lt : 0, r);
        if (ltile < ntiles) advance(ltile, lt);
    };
    // the first weight loads go out before the staging
    load_next(buf[0]);
    {
        const XT* xcol[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xcol[b] = x + b * ldx;
        q4k_stage_x<B, 64 * NW, XT>(xcol, 256 * nsb, xs, xvec != 0);   // ends with a barrier
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

template <int B, int LPR, int NW, class XT>
int32_t q4k_launch(const uint8_t* W, int64_t N, int nsb, const XT* x, int64_t ldx, float* y, int64_t ldy,
                   hipStream_t st) {
    auto kern = q4k_kernel<B, LPR, NW, XT>;
    const size_t lds = (size_t)B * 4 * nsb * kQ4KXPad * sizeof(float);
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv_q4_k", &dyn_max)) return e;
    if (lds > dyn_max) return fail(QMV_EINVAL, "qmv_q4_k: %zu bytes of staged activations exceed the LDS", lds);
    constexpr int rows_per_wg = NW * (64 / LPR);
    const int64_t tiles = (N + rows_per_wg - 1) / rows_per_wg;
    const int per_cu = std::max(1, resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds));
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, (int64_t)device_cu_count() * per_cu));
    const int xvec = (aligned(x, XIn<XT>::kVecAlign) && ldx % 4 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, W, N, nsb, x, ldx, y, ldy, xvec);
    return check_launch("qmv_q4_k");
}

// Lanes per row: the widest split of 64 / 32 / 16 / 8 lanes that leaves at
// most 1/16 of a row's lane-steps idle (wide splits keep more waves busy on
// matrices of few rows), else the split with the fewest idle: 64 for 4096
// columns (64 groups of 64 weights), 32 for 14336 (224 groups: 7 full
// steps, where whole waves would leave half of the fourth step idle), 16
// for 3072 (48 groups).
inline int q4k_pick_lpr(int G) {
    int best = 8;
    int64_t best_idle = 1 << 30, best_span = 1;
    for (const int l : {64, 32, 16, 8}) {
        if (l > G && l != 8) continue;
        const int64_t span = (G + l - 1) / l * l;   // lane-steps per row
        const int64_t idle = span - G;
        if (16 * idle <= span) return l;
        if (idle * best_span < best_idle * span) {  // idle / span, exactly
            best = l;
            best_idle = idle;
            best_span = span;
        }
    }
    return best;
}

template <int B, int NW, class XT>
int32_t q4k_launch_lpr(const uint8_t* W, int64_t N, int nsb, const XT* x, int64_t ldx, float* y, int64_t ldy,
                       hipStream_t st) {
    switch (q4k_pick_lpr(4 * nsb)) {
    case 64: return q4k_launch<B, 64, NW, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 32: return q4k_launch<B, 32, NW, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 16: return q4k_launch<B, 16, NW, XT>(W, N, nsb, x, ldx, y, ldy, st);
    default: return q4k_launch<B, 8, NW, XT>(W, N, nsb, x, ldx, y, ldy, st);
    }
}

template <class XT>
int32_t q4k_batch(const uint8_t* W, int64_t N, int nsb, const XT* x, int64_t ldx, int B, float* y, int64_t ldy,
                  hipStream_t st) {
    switch (B) {
    case 1: return q4k_launch_lpr<1, 8, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 2: return q4k_launch_lpr<2, 8, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 3: return q4k_launch_lpr<3, 8, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 4: return q4k_launch_lpr<4, 8, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 5: return q4k_launch_lpr<5, 8, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 6: return q4k_launch_lpr<6, 8, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 7: return q4k_launch_lpr<7, 8, XT>(W, N, nsb, x, ldx, y, ldy, st);
    default: return q4k_launch_lpr<8, 8, XT>(W, N, nsb, x, ldx, y, ldy, st);
    }
}

template <class XT>
int32_t q4k_matvec_t(const char* name, const void* W, int64_t N, int64_t K, const XT* x, int32_t x_type, int64_t ldx,
                     int32_t batch, float* y, int64_t ldy, void* stream, int32_t path) {
    if (!W || !x || !y) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (N < 1) return fail(QMV_EINVAL, "%s: n_rows must be >= 1 (got %lld)", name, (long long)N);
    if (K < kQ4KWeights || K % kQ4KWeights)
        return fail(QMV_EINVAL, "%s: n_cols must be a positive multiple of 256 for Q4_K (got %lld)", name,
                    (long long)K);
    if (batch < 1 || batch > 8) return fail(QMV_EINVAL, "%s: batch must be in 1..8 (got %d)", name, batch);
    if (ldx < K) return fail(QMV_EINVAL, "%s: ldx (%lld) < n_cols (%lld)", name, (long long)ldx, (long long)K);
    if (ldy < N) return fail(QMV_EINVAL, "%s: ldy (%lld) < n_rows (%lld)", name, (long long)ldy, (long long)N);
    if (K / kQ4KWeights > (1 << 24) || N > ((int64_t)1 << 40) / (K / kQ4KWeights))
        return fail(QMV_EINVAL, "%s: matrix too large (%lld x %lld)", name, (long long)N, (long long)K);
    if (!aligned(W, 16)) return fail(QMV_EALIGN, "%s: W must be 16-byte aligned for Q4_K", name);
    if (!aligned(y, 4)) return fail(QMV_EALIGN, "%s: y must be 4-byte aligned", name);
    if (!aligned(x, sizeof(XT))) return fail(QMV_EALIGN, "%s: x must be aligned to its element size", name);
    const int nsb = (int)(K / kQ4KWeights);
    // Batch 3..8 on the matrix cores (codes about a pivot per sub-block and
    // block sums of x, as for Q4_1), where the shape allows.
    if (path == QMV_PATH_MFMA || (path == QMV_PATH_AUTO && use_mfma(QMV_Q4_K, N, 8 * nsb, batch))) {
        int32_t rc = QMV_OK;
        if (batch_matvec_mma(QMV_Q4_K, static_cast<const uint8_t*>(W), N, 8 * nsb, x, x_type, ldx, batch, y, ldy,
                             as_stream(stream), 0, &rc))
            return rc == QMV_OK ? ok() : rc;
        if (path == QMV_PATH_MFMA)
            return fail(QMV_EUNSUPPORTED,
                        "%s: the matrix-core path needs batch 2..8, x aligned to 4 elements (16 bytes for fp32) and "
                        "ldx a multiple of 4", name);
    }
    const int per_col = 4 * nsb * kQ4KXPad * (int)sizeof(float);
    if (per_col > kLdsMax)
        return fail(QMV_EINVAL, "%s: n_cols %lld too large for one activation row in LDS", name, (long long)K);
    const int per_pass = std::max(1, std::min<int>(batch, kLdsMax / per_col));
    for (int b0 = 0; b0 < batch; b0 += per_pass) {
        const int bw = std::min(per_pass, batch - b0);
        const int32_t rc = q4k_batch<XT>(static_cast<const uint8_t*>(W), N, nsb, x + b0 * ldx, ldx, bw,
                                         y + b0 * ldy, ldy, as_stream(stream));
        if (rc != QMV_OK) return rc;
    }
    return ok();
}

int32_t q4k_matvec(const char* name, const void* W, int64_t N, int64_t K, const void* x, int32_t x_type, int64_t ldx,
                   int32_t batch, float* y, int64_t ldy, void* stream, int32_t path) {
    switch (x_type) {
    case QMV_X_F32:
        return q4k_matvec_t(name, W, N, K, static_cast<const float*>(x), x_type, ldx, batch, y, ldy, stream, path);
    case QMV_X_F16:
        return q4k_matvec_t(name, W, N, K, static_cast<const _Float16*>(x), x_type, ldx, batch, y, ldy, stream, path);
    case QMV_X_BF16:
        return q4k_matvec_t(name, W, N, K, static_cast<const __bf16*>(x), x_type, ldx, batch, y, ldy, stream, path);
    default: return fail(QMV_EINVAL, "%s: unknown x_type %d", name, (int)x_type);
    }
}

int32_t q4k_dequant(const void* W, int64_t N, int64_t K, float* out, void* stream) {
    const char* name = "qmv_dequant";
    if (!W || !out) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (N < 1) return fail(QMV_EINVAL, "%s: n_rows must be >= 1 (got %lld)", name, (long long)N);
    if (K < kQ4KWeights || K % kQ4KWeights)
        return fail(QMV_EINVAL, "%s: n_cols must be a positive multiple of 256 for Q4_K (got %lld)", name,
                    (long long)K);
    if (N > ((int64_t)1 << 40) / K) return fail(QMV_EINVAL, "%s: matrix too large", name);
    if (!aligned(W, 16) || !aligned(out, 4)) return fail(QMV_EALIGN, "%s: W must be 16-byte aligned for Q4_K", name);
    const int64_t nsub = N * (K / 32);
    const int64_t grid = (nsub + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(q4k_dequant_kernel, dim3((unsigned)grid), dim3(kThreads), 0, as_stream(stream),
                       static_cast<const uint8_t*>(W), nsub, out);
    return check_launch(name);
}

int32_t q4k_no_moe(const char* name, bool, const void*, int64_t, int32_t, int64_t, int64_t, const int32_t*, int32_t,
                   int32_t, const void*, int32_t, int64_t, int64_t, float*, void*) {
    return fail(QMV_EUNSUPPORTED, "%s: Q4_K experts are not supported", name);
}
int32_t q4k_no_combine(const void*, int64_t, int32_t, int64_t, int64_t, const int32_t*, const float*, int32_t, int32_t,
                       const float*, int64_t, int64_t, float*, void*) {
    return fail(QMV_EUNSUPPORTED, "qmv_moe_combine: Q4_K experts are not supported");
}
bool q4k_no_group(const RowSegs&, int, const float*, hipStream_t, bool, int32_t*) { return false; }

}  // namespace

const FormatOps& ops_q4_k() {
    static const FormatOps ops = {q4k_matvec, q4k_dequant, q4k_no_moe, q4k_no_combine, q4k_no_group};
    return ops;
}

}  // namespace qmv

extern "C" int32_t qmv_q4_k(const void* W, int64_t n_rows, int64_t n_cols, const float* x, int64_t ldx, int32_t batch,
                            float* y, int64_t ldy, void* stream) {
    return qmv::ops_q4_k().matvec("qmv_q4_k", W, n_rows, n_cols, x, QMV_X_F32, ldx, batch, y, ldy, stream,
                                  QMV_PATH_AUTO);
}
