// Pieces shared by the super-block formats (256 weights per super-block,
// one lane per 64-weight group of a row): activation staging into LDS, the
// lanes-per-row rule, and the host side of a matvec (argument checks,
// column passes, launch shape, the matrix-core hand-off) and of the
// dequantizer.  A format supplies a traits struct Fmt:
//   kFmt            its qmv_fmt (for the matrix-core hand-off, when kMfma)
//   kLabel          "Q4_K", "Q6_K" (error messages)
//   kEntry          the C entry point's name (launch error messages)
//   kWAlign         alignment W needs, in bytes
//   kMfma           whether batch 2..8 may go to the matrix-core kernel
//   kDequantWeights weights per thread of its dequant kernel
//   kBytes          bytes per super-block
//   template <int B, int LPR, int NW, class XT, bool ROUTE> static auto kernel()
//                   the matvec kernel: (W, N, nsb, x, ldx, y, ldy, xvec,
//                   route), with LDS for B activation rows at kSbXPad floats
//                   per 64 weights; ROUTE: grid row p computes MoE pair p
//                   (SbRoute)
//   static auto dequant_kernel()   (W, n_units, out), one unit per thread
#pragma once

#include <algorithm>

#include "qmv_block_decode.h"

namespace qmv {
namespace {

constexpr int kSbWeights = 256;   // per super-block
constexpr int kSbMaxSlots = 16;   // top_k of the MoE entry points
constexpr int kSbCombineRows = 1024;   // rows per workgroup of a combine launch, at most

// MoE routing of the super-block kernels: grid row p = b * top_k + s
// (blockIdx.y) computes y[p] = DEQ(W_e) x_{b,s} with e = ids[p], x_{b,s} at
// x + b * xs_tok + s * xs_slot (elements) and y[p] at y + p * ldy.  An id
// outside [0, n_experts) streams expert 0 and writes quiet NaN.
struct SbRoute {
    const int32_t* ids;
    int64_t estride;              // bytes between experts
    int64_t xs_tok, xs_slot;
    int32_t top_k, n_experts;
};

// Applies the route of grid row blockIdx.y to the kernel's W, x and y
// pointers; returns whether its id is bad.
template <class PW, class PX, class PY>
__device__ __forceinline__ bool sb_route(const SbRoute& route, PW& W, PX& x, PY& y, int64_t ldy) {
    const int p = blockIdx.y;
    const int e = route.ids[p];            // uniform: one scalar load
    const bool bad = e < 0 || e >= route.n_experts;
    W += (int64_t)(bad ? 0 : e) * route.estride;
    x += (int64_t)(p / route.top_k) * route.xs_tok + (int64_t)(p % route.top_k) * route.xs_slot;
    y += (int64_t)p * ldy;
    return bad;
}
constexpr int kSbXPad = 68;       // staged floats per 64-weight lane group: 16-byte reads of
                                  // lanes on consecutive groups start 4 banks apart

// Hides a value's bits from the optimizer: a masked word then converts with
// one byte-select convert per element instead of a bit-field extract and a
// convert.
__device__ __forceinline__ uint32_t opaque_bits(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// Stages the B columns xcol[b][0..K) into LDS as fp32 (16-bit inputs
// widened exactly), element e of column b at xs[b * (K / 64) * kSbXPad +
// slot(e)]; slot maps 4-aligned runs of 4 elements to 16-byte-aligned runs.
// Loads in batches of 4 per thread before any is stored; vec: every column
// aligned for 4-element loads.  Ends with a barrier.
template <int B, int NT, class XT, class Slot>
__device__ __forceinline__ void sb_stage_x(const XT* const (&xcol)[B], int K, float* xs, bool vec, Slot slot) {
    const int G = K >> 6;
    const int tid = threadIdx.x;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float* dst = xs + b * G * kSbXPad;
        const XT* src = xcol[b];
        if (vec) {
            const int K4 = K >> 2;
            auto put = [&](int c, const float4& v) { *reinterpret_cast<float4*>(dst + slot(4 * c)) = v; };
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
            for (int e0 = tid; e0 < K; e0 += 4 * NT) {
                const int e1 = e0 + NT, e2 = e0 + 2 * NT, e3 = e0 + 3 * NT;
                const float v0 = XIn<XT>::load1(src + e0);
                const float v1 = XIn<XT>::load1(src + min(e1, K - 1));
                const float v2 = XIn<XT>::load1(src + min(e2, K - 1));
                const float v3 = XIn<XT>::load1(src + min(e3, K - 1));
                dst[slot(e0)] = v0;
                if (e1 < K) dst[slot(e1)] = v1;
                if (e2 < K) dst[slot(e2)] = v2;
                if (e3 < K) dst[slot(e3)] = v3;
            }
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------- kernels
// over one format's batch-1 step.  Ops (per format) provides:
//   Raw                      the stored bytes one lane loads for one step
//   kBytes                   bytes per super-block
//   fetch(row, g, r)         loads group g (64 weights) of the row at `row`
//   group_sum(r, li, gc, xs) the group's sum for one column staged at xs:
//                            bitwise the batch-1 kernel's step sum
//   slot(e)                  the LDS float index of activation element e
//   kWaves                   waves per SIMD the kernels are held to (1: the
//                            compiler's choice)
// A lane li of a segment of LPR lanes takes group li + LPR t of its row in
// step t and a row's sum is the segment's, as in the batch-1 kernels, so
// these kernels' row sums are bitwise theirs.

// Up to kMaxSegs matrices of one width that read one x (decode's q, k and
// v), as one batch-1 launch over their concatenated rows: a lane's row
// picks its matrix from the cumulative row counts (constant indices only,
// so the table stays in registers).
template <class Ops, int LPR, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(Ops::kWaves))) void sb_group_kernel(
    const RowSegs segs, int nsb, const float* __restrict__ x, int xvec) {
    using Raw = typename Ops::Raw;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* xs = lds;                          // [4 nsb][kSbXPad]
    constexpr int RW = 64 / LPR;              // rows per tile
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int G = 4 * nsb;
    const int T = (G + LPR - 1) / LPR;
    const int64_t pitch = (int64_t)nsb * Ops::kBytes;
    const int64_t rows = segs.end[segs.n - 1];
    const int64_t ntiles = (rows + RW - 1) / RW;
    const int64_t wstride = (int64_t)gridDim.x * NW;
    auto locate = [&](int64_t row, const uint8_t*& Wm, float*& ym, int64_t& start) {
        Wm = segs.W[0];
        ym = segs.y[0];
        start = 0;
#pragma unroll
        for (int i = 1; i < kMaxSegs; ++i) {
            const bool in = i < segs.n && row >= segs.end[i - 1];
            Wm = in ? segs.W[i] : Wm;
            ym = in ? segs.y[i] : ym;
            start = in ? segs.end[i - 1] : start;
        }
    };
    auto load_step = [&](int64_t tile, int t, Raw& r) {
        const int g = min(li + LPR * t, G - 1);                 // clamp: stays in bounds
        const int64_t row = min(tile * RW + seg, rows - 1);     // rows past the end: the last row
        const uint8_t* Wm;
        float* ym;
        int64_t start;
        locate(row, Wm, ym, start);
        Ops::fetch(Wm + (row - start) * pitch, g, r);
    };
    float acc = 0.f;
    auto compute_step = [&](int64_t tile, int t, const Raw& r) {
        const int g = li + LPR * t;
        const bool valid = g < G;
        const int gc = valid ? g : G - 1;
        const float s = Ops::group_sum(r, li, gc, xs);
        acc = valid ? acc + s : acc;
        if (t == T - 1) {
            const float tot = segment_sum<LPR>(acc);
            const int64_t row = tile * RW + seg;
            if (li == 0 && row < rows) {
                const uint8_t* Wm;
                float* ym;
                int64_t start;
                locate(row, Wm, ym, start);
                ym[row - start] = tot;
            }
            acc = 0.f;
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
    Raw buf[2];
    auto load_next = [&](Raw& r) {
        load_step(min(ltile, ntiles - 1), ltile < ntiles ? lt : 0, r);
        if (ltile < ntiles) advance(ltile, lt);
    };
    load_next(buf[0]);
    {
        const float* xcol[1] = {x};
        sb_stage_x<1, 64 * NW, float>(xcol, kSbWeights * nsb, xs, xvec != 0, Ops::slot);   // ends with a barrier
    }
    // two register buffers used in turn; once the load cursor is past the
    // wave's last step, the step in hand is computed after the loop
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

// MoE down projection with the router-weighted combine, token-major:
// workgroup (bx, b) computes rows [r0, r1) of out[b] = sum_s w[b][s] *
// DEQ(W_{e_s}) x_{b,s} over the top_k slots of token b.  The slots'
// activation vectors are staged together (SC at a time when they do not all
// fit the LDS).  The work is the units (slot, tile of RW rows); wave w takes
// units w, w + NW, ... with a two-deep load pipeline across them, and each
// unit's row sums (bitwise the qmv_moe outputs) go to LDS.  Then one thread
// per row adds them in slot order, fma(w_s, y_s, acc) from s = 0 up.  An
// expert routed from several tokens is read once per token (no atomics, no
// workspace).
template <class Ops, int LPR, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(Ops::kWaves))) void sb_combine_kernel(
    const uint8_t* __restrict__ Wx, int64_t estride, int n_experts, int64_t N, int nsb,
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int top_k, const float* __restrict__ x,
    int64_t xs_tok, int64_t xs_slot, float* __restrict__ out, int xvec, int SC, int rows_wg) {
    using Raw = typename Ops::Raw;
    __shared__ const uint8_t* s_base[kSbMaxSlots];
    __shared__ float s_w[kSbMaxSlots];
    __shared__ int s_bad;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int RW = 64 / LPR;              // rows per tile
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int G = 4 * nsb;                    // 64-weight groups per row
    const int T = (G + LPR - 1) / LPR;        // steps per row
    const int64_t pitch = (int64_t)nsb * Ops::kBytes;
    const int b = blockIdx.y;
    const int64_t ntiles = (N + RW - 1) / RW;
    const int per_wg = rows_wg / RW;
    const int64_t tb = (int64_t)blockIdx.x * per_wg;
    const int64_t te = min(ntiles, tb + per_wg);
    if (tb >= te) return;                     // the whole workgroup: no barrier is skipped by part of it
    const int wtiles = (int)(te - tb);
    const int per_col = G * kSbXPad;          // floats of one staged slot vector
    float* xs = lds;                          // [SC][G][kSbXPad]
    float* ybuf = lds + SC * per_col;         // [top_k][rows_wg]: row sums per slot
    const int64_t r0 = tb * RW;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    if (tid < top_k) {
        const int e = ids[b * top_k + tid];
        const bool eb = e < 0 || e >= n_experts;
        if (eb) s_bad = 1;
        s_base[tid] = Wx + (int64_t)(eb ? 0 : e) * estride;
        s_w[tid] = wts[b * top_k + tid];
    }
    __syncthreads();                          // s_base, s_w, s_bad
    for (int s0 = 0; s0 < top_k; s0 += SC) {
        const int sc = min(SC, top_k - s0);
        const int units = sc * wtiles;
        const int my_units = wave < units ? (units - wave + NW - 1) / NW : 0;
        const int nsteps = my_units * T;
        // the chunk's slot vectors (every wave is done with the previous
        // chunk's: its units all ended before this barrier)
        __syncthreads();
        for (int k = 0; k < sc; ++k) {
            const float* xcol[1] = {x + (int64_t)b * xs_tok + (int64_t)(s0 + k) * xs_slot};
            sb_stage_x<1, 64 * NW, float>(xcol, kSbWeights * nsb, xs + k * per_col, xvec != 0, Ops::slot);
        }
        if (nsteps == 0) continue;
        // step n of this wave: unit q = wave + NW (n / T), group step t = n % T
        auto load = [&](int n, Raw& r) {
            const int q = wave + NW * (n / T);
            const int t = n % T;
            const int slot = q / wtiles;
            const int64_t tile = tb + (q - slot * wtiles);
            const int g = min(li + LPR * t, G - 1);             // clamp: stays in bounds
            const int64_t rt = tile * RW;                        // tile < ntiles: rt < N
            const int64_t rem = N - 1 - rt;
            const int lr = min(seg, rem < RW - 1 ? (int)rem : RW - 1);   // rows past the end: the last row
            Ops::fetch(s_base[s0 + slot] + (rt + lr) * pitch, g, r);
        };
        float acc = 0.f;
        auto compute = [&](int n, const Raw& r) {
            const int q = wave + NW * (n / T);
            const int t = n % T;
            const int slot = q / wtiles;
            const int64_t tile = tb + (q - slot * wtiles);
            const int g = li + LPR * t;
            const bool valid = g < G;
            const int gc = valid ? g : G - 1;
            const float s = Ops::group_sum(r, li, gc, xs + slot * per_col);
            acc = valid ? acc + s : acc;
            if (t == T - 1) {
                const float tot = segment_sum<LPR>(acc);
                const int64_t row = tile * RW + seg;
                if (li == 0 && row < N) ybuf[(s0 + slot) * rows_wg + (row - r0)] = tot;
                acc = 0.f;
            }
        };
        // two register buffers used in turn (nsteps is wave-uniform)
        Raw buf0, buf1;
        load(0, buf0);
        for (int n = 0;;) {
            if (n + 1 < nsteps) load(n + 1, buf1);
            __builtin_amdgcn_sched_barrier(0);
            compute(n, buf0);
            if (++n == nsteps) break;
            if (n + 1 < nsteps) load(n + 1, buf0);
            __builtin_amdgcn_sched_barrier(0);
            compute(n, buf1);
            if (++n == nsteps) break;
        }
    }
    __syncthreads();
    const float qnan = __builtin_nanf("");
    const int64_t r1 = min(te * RW, N);
    for (int64_t row = r0 + tid; row < r1; row += 64 * NW) {
        const float* yr = ybuf + (row - r0);
        float v = s_w[0] * yr[0];
        for (int s = 1; s < top_k; ++s) v = __builtin_fmaf(s_w[s], yr[s * rows_wg], v);
        out[(int64_t)b * N + row] = s_bad ? qnan : v;
    }
}

// MoE gate||up with SwiGLU fused, one grid row per (token, slot) pair (as
// the batch-1 kernels' routed form): every expert holds 2N rows, gate rows
// then up rows, and the segment of output row i streams gate row i and up
// row N + i in the same lanes and steps, then writes SiLU(gate) * up.  Each
// row's sum is the batch-1 kernel's.
template <class Ops, int LPR, int NW, class XT>
__global__ __launch_bounds__(64 * NW) void sb_swiglu_kernel(const uint8_t* __restrict__ W, int64_t N, int nsb,
                                                             const XT* __restrict__ x, int64_t ldx,
                                                             float* __restrict__ y, int64_t ldy, int xvec,
                                                             const SbRoute route) {
    using Raw = typename Ops::Raw;
    const bool bad = sb_route(route, W, x, y, ldy);
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* xs = lds;                          // [4 nsb][kSbXPad]
    constexpr int RW = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int G = 4 * nsb;
    const int T = (G + LPR - 1) / LPR;
    const int64_t pitch = (int64_t)nsb * Ops::kBytes;
    const int64_t ntiles = (N + RW - 1) / RW;
    const int64_t wstride = (int64_t)gridDim.x * NW;
    struct Pair {
        Raw g, u;
    };
    auto load_step = [&](int64_t tile, int t, Pair& r) {
        const int g = min(li + LPR * t, G - 1);                 // clamp: stays in bounds
        const int64_t row = min(tile * RW + seg, N - 1);        // rows past the end: the last row
        Ops::fetch(W + row * pitch, g, r.g);
        Ops::fetch(W + (N + row) * pitch, g, r.u);
    };
    float acc_g = 0.f, acc_u = 0.f;
    auto compute_step = [&](int64_t tile, int t, const Pair& r) {
        const int g = li + LPR * t;
        const bool valid = g < G;
        const int gc = valid ? g : G - 1;
        const float sg = Ops::group_sum(r.g, li, gc, xs);
        const float su = Ops::group_sum(r.u, li, gc, xs);
        acc_g = valid ? acc_g + sg : acc_g;
        acc_u = valid ? acc_u + su : acc_u;
        if (t == T - 1) {
            const float gs = segment_sum<LPR>(acc_g);
            const float us = segment_sum<LPR>(acc_u);
            const int64_t row = tile * RW + seg;
            if (li == 0 && row < N) y[row] = bad ? __builtin_nanf("") : silu(gs) * us;
            acc_g = acc_u = 0.f;
        }
    };
    auto advance = [&](int64_t& tile, int& t) {
        if (++t == T) {
            t = 0;
            tile += wstride;
        }
    };
    int64_t ltile = (int64_t)blockIdx.x * NW + wave;
    int lt = 0;
    int64_t ctile = ltile;
    int ct = 0;
    Pair buf[2];
    auto load_next = [&](Pair& r) {
        load_step(min(ltile, ntiles - 1), ltile < ntiles ? lt : 0, r);
        if (ltile < ntiles) advance(ltile, lt);
    };
    load_next(buf[0]);
    {
        const XT* xcol[1] = {x};
        sb_stage_x<1, 64 * NW, XT>(xcol, kSbWeights * nsb, xs, xvec != 0, Ops::slot);   // ends with a barrier
    }
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

// Lanes per row: the widest split of 64 / 32 / 16 / 8 lanes that leaves at
// most 1/16 of a row's lane-steps idle (wide splits keep more waves busy on
// matrices of few rows), else the split with the fewest idle: 64 for 4096
// columns (64 groups of 64 weights), 32 for 14336 (224 groups: 7 full
// steps, where whole waves would leave half of the fourth step idle), 16
// for 3072 (48 groups).
inline int sb_pick_lpr(int G) {
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

// route: MoE pairs (grid rows) or nullptr (one dense matrix).  SW (routed
// only): N output rows of SiLU(gate) * up from experts of 2N rows.
template <class Fmt, int B, int LPR, int NW, class XT, bool SW = false>
int32_t sb_launch(const uint8_t* W, int64_t N, int nsb, const XT* x, int64_t ldx, float* y, int64_t ldy,
                  hipStream_t st, const SbRoute* route, int pairs) {
    if (route) {
        if constexpr (B == 1) {
            auto kern = [] {
                if constexpr (SW) return Fmt::template swiglu_kernel<LPR, NW, XT>();
                else return Fmt::template kernel<1, LPR, NW, XT, true>();
            }();
            const size_t lds = (size_t)4 * nsb * kSbXPad * sizeof(float);
            size_t dyn_max = 0;
            if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, Fmt::kEntry, &dyn_max))
                return e;
            if (lds > dyn_max)
                return fail(QMV_EINVAL, "%s: %zu bytes of staged activations exceed the LDS", Fmt::kEntry, lds);
            constexpr int rows_per_wg = NW * (64 / LPR);
            const int64_t tiles = (N + rows_per_wg - 1) / rows_per_wg;
            const int per_cu = std::max(1, resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds));
            const int64_t slots = std::max<int64_t>(1, (int64_t)device_cu_count() * per_cu / pairs);
            const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, slots));
            const int xvec = (aligned(x, XIn<XT>::kVecAlign) && route->xs_tok % 4 == 0 && route->xs_slot % 4 == 0)
                                 ? 1 : 0;
            hipLaunchKernelGGL(kern, dim3(grid, pairs), dim3(64 * NW), lds, st, W, N, nsb, x, ldx, y, ldy, xvec,
                               *route);
            return check_launch(Fmt::kEntry);
        } else {
            return fail(QMV_EINVAL, "%s: routed launches take one column", Fmt::kEntry);
        }
    }
    auto kern = Fmt::template kernel<B, LPR, NW, XT, false>();
    const size_t lds = (size_t)B * 4 * nsb * kSbXPad * sizeof(float);
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, Fmt::kEntry, &dyn_max)) return e;
    if (lds > dyn_max) return fail(QMV_EINVAL, "%s: %zu bytes of staged activations exceed the LDS", Fmt::kEntry, lds);
    constexpr int rows_per_wg = NW * (64 / LPR);
    const int64_t tiles = (N + rows_per_wg - 1) / rows_per_wg;
    const int per_cu = std::max(1, resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds));
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, (int64_t)device_cu_count() * per_cu));
    const int xvec = (aligned(x, XIn<XT>::kVecAlign) && ldx % 4 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, W, N, nsb, x, ldx, y, ldy, xvec, SbRoute{});
    return check_launch(Fmt::kEntry);
}

// 8 waves per workgroup at every batch width (a workgroup of 16 would cap
// the registers at 128, and batch 6..8 need more).
template <class Fmt, int B, class XT, bool SW = false>
int32_t sb_launch_lpr(const uint8_t* W, int64_t N, int nsb, const XT* x, int64_t ldx, float* y, int64_t ldy,
                      hipStream_t st, const SbRoute* route = nullptr, int pairs = 1) {
    switch (sb_pick_lpr(4 * nsb)) {
    case 64: return sb_launch<Fmt, B, 64, 8, XT, SW>(W, N, nsb, x, ldx, y, ldy, st, route, pairs);
    case 32: return sb_launch<Fmt, B, 32, 8, XT, SW>(W, N, nsb, x, ldx, y, ldy, st, route, pairs);
    case 16: return sb_launch<Fmt, B, 16, 8, XT, SW>(W, N, nsb, x, ldx, y, ldy, st, route, pairs);
    default: return sb_launch<Fmt, B, 8, 8, XT, SW>(W, N, nsb, x, ldx, y, ldy, st, route, pairs);
    }
}

template <class Fmt, class XT>
int32_t sb_batch(const uint8_t* W, int64_t N, int nsb, const XT* x, int64_t ldx, int B, float* y, int64_t ldy,
                 hipStream_t st) {
    switch (B) {
    case 1: return sb_launch_lpr<Fmt, 1, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 2: return sb_launch_lpr<Fmt, 2, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 3: return sb_launch_lpr<Fmt, 3, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 4: return sb_launch_lpr<Fmt, 4, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 5: return sb_launch_lpr<Fmt, 5, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 6: return sb_launch_lpr<Fmt, 6, XT>(W, N, nsb, x, ldx, y, ldy, st);
    case 7: return sb_launch_lpr<Fmt, 7, XT>(W, N, nsb, x, ldx, y, ldy, st);
    default: return sb_launch_lpr<Fmt, 8, XT>(W, N, nsb, x, ldx, y, ldy, st);
    }
}

template <class Fmt, class XT>
int32_t sb_matvec_t(const char* name, const void* W, int64_t N, int64_t K, const XT* x, int32_t x_type, int64_t ldx,
                    int32_t batch, float* y, int64_t ldy, void* stream, int32_t path) {
    if (!W || !x || !y) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (N < 1) return fail(QMV_EINVAL, "%s: n_rows must be >= 1 (got %lld)", name, (long long)N);
    if (K < kSbWeights || K % kSbWeights)
        return fail(QMV_EINVAL, "%s: n_cols must be a positive multiple of 256 for %s (got %lld)", name, Fmt::kLabel,
                    (long long)K);
    if (batch < 1 || batch > 8) return fail(QMV_EINVAL, "%s: batch must be in 1..8 (got %d)", name, batch);
    if (ldx < K) return fail(QMV_EINVAL, "%s: ldx (%lld) < n_cols (%lld)", name, (long long)ldx, (long long)K);
    if (ldy < N) return fail(QMV_EINVAL, "%s: ldy (%lld) < n_rows (%lld)", name, (long long)ldy, (long long)N);
    if (K / kSbWeights > (1 << 24) || N > ((int64_t)1 << 40) / (K / kSbWeights))
        return fail(QMV_EINVAL, "%s: matrix too large (%lld x %lld)", name, (long long)N, (long long)K);
    if (!aligned(W, Fmt::kWAlign))
        return fail(QMV_EALIGN, "%s: W must be %d-byte aligned for %s", name, Fmt::kWAlign, Fmt::kLabel);
    if (!aligned(y, 4)) return fail(QMV_EALIGN, "%s: y must be 4-byte aligned", name);
    if (!aligned(x, sizeof(XT))) return fail(QMV_EALIGN, "%s: x must be aligned to its element size", name);
    const int nsb = (int)(K / kSbWeights);
    if constexpr (Fmt::kMfma) {
        if (path == QMV_PATH_MFMA || (path == QMV_PATH_AUTO && use_mfma(Fmt::kFmt, N, 8 * nsb, batch))) {
            int32_t rc = QMV_OK;
            if (batch_matvec_mma(Fmt::kFmt, static_cast<const uint8_t*>(W), N, 8 * nsb, x, x_type, ldx, batch, y,
                                 ldy, as_stream(stream), 0, &rc))
                return rc == QMV_OK ? ok() : rc;
            if (path == QMV_PATH_MFMA)
                return fail(QMV_EUNSUPPORTED,
                            "%s: the matrix-core path needs batch 2..8, x aligned to 4 elements (16 bytes for fp32) "
                            "and ldx a multiple of 4", name);
        }
    } else {
        if (path == QMV_PATH_MFMA)
            return fail(QMV_EUNSUPPORTED, "%s: %s has no matrix-core kernel (use QMV_PATH_AUTO or QMV_PATH_FMA)", name,
                        Fmt::kLabel);
    }
    // One activation row per column must fit the LDS; wider batches than
    // fit go in column passes (each re-reads W).
    const int per_col = 4 * nsb * kSbXPad * (int)sizeof(float);
    if (per_col > kLdsMax)
        return fail(QMV_EINVAL, "%s: n_cols %lld too large for one activation row in LDS", name, (long long)K);
    const int per_pass = std::max(1, std::min<int>(batch, kLdsMax / per_col));
    for (int b0 = 0; b0 < batch; b0 += per_pass) {
        const int bw = std::min(per_pass, batch - b0);
        const int32_t rc = sb_batch<Fmt, XT>(static_cast<const uint8_t*>(W), N, nsb, x + b0 * ldx, ldx, bw,
                                             y + b0 * ldy, ldy, as_stream(stream));
        if (rc != QMV_OK) return rc;
    }
    return ok();
}

template <class Fmt>
int32_t sb_matvec(const char* name, const void* W, int64_t N, int64_t K, const void* x, int32_t x_type, int64_t ldx,
                  int32_t batch, float* y, int64_t ldy, void* stream, int32_t path) {
    switch (x_type) {
    case QMV_X_F32:
        return sb_matvec_t<Fmt>(name, W, N, K, static_cast<const float*>(x), x_type, ldx, batch, y, ldy, stream, path);
    case QMV_X_F16:
        return sb_matvec_t<Fmt>(name, W, N, K, static_cast<const _Float16*>(x), x_type, ldx, batch, y, ldy, stream,
                                path);
    case QMV_X_BF16:
        return sb_matvec_t<Fmt>(name, W, N, K, static_cast<const __bf16*>(x), x_type, ldx, batch, y, ldy, stream,
                                path);
    default: return fail(QMV_EINVAL, "%s: unknown x_type %d", name, (int)x_type);
    }
}

template <class Fmt>
int32_t sb_dequant(const void* W, int64_t N, int64_t K, float* out, void* stream) {
    const char* name = "qmv_dequant";
    if (!W || !out) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (N < 1) return fail(QMV_EINVAL, "%s: n_rows must be >= 1 (got %lld)", name, (long long)N);
    if (K < kSbWeights || K % kSbWeights)
        return fail(QMV_EINVAL, "%s: n_cols must be a positive multiple of 256 for %s (got %lld)", name, Fmt::kLabel,
                    (long long)K);
    if (N > ((int64_t)1 << 40) / K) return fail(QMV_EINVAL, "%s: matrix too large", name);
    if (!aligned(W, Fmt::kWAlign))
        return fail(QMV_EALIGN, "%s: W must be %d-byte aligned for %s", name, Fmt::kWAlign, Fmt::kLabel);
    if (!aligned(out, 4)) return fail(QMV_EALIGN, "%s: out must be 4-byte aligned", name);
    const int64_t units = N * (K / Fmt::kDequantWeights);
    const int64_t grid = (units + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(Fmt::dequant_kernel(), dim3((unsigned)grid), dim3(kThreads), 0, as_stream(stream),
                       static_cast<const uint8_t*>(W), units, out);
    return check_launch(name);
}

// MoE experts: every (token, slot) pair is one grid row of the batch-1
// kernel (a pair's expert is streamed for that pair; an expert shared by
// several pairs is read from HBM about once, its other reads hitting the
// caches).  SW: the fused SwiGLU form, N output rows per pair from experts
// of 2N rows (formats whose kernel has it).
template <class Fmt, class XT, bool SW = false>
int32_t sb_moe_t(const char* name, const void* Wx, int64_t estride, int32_t E, int64_t N, int64_t K,
                 const int32_t* ids, int32_t batch, int32_t top_k, const XT* x, int64_t xs_tok, int64_t xs_slot,
                 float* y, void* stream) {
    if (!Wx || !ids || !x || !y) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (E < 1) return fail(QMV_EINVAL, "%s: n_experts must be >= 1", name);
    if (N < 1 || K < kSbWeights || K % kSbWeights)
        return fail(QMV_EINVAL, "%s: bad matrix shape %lld x %lld (n_cols a multiple of 256 for %s)", name,
                    (long long)N, (long long)K, Fmt::kLabel);
    if (batch < 1 || batch > 8) return fail(QMV_EINVAL, "%s: batch must be in 1..8 (got %d)", name, batch);
    if (top_k < 1 || top_k > 16) return fail(QMV_EINVAL, "%s: top_k must be in 1..16 (got %d)", name, top_k);
    const int64_t nsb = K / kSbWeights;
    if (SW && N > ((int64_t)1 << 39)) return fail(QMV_EINVAL, "%s: n_ff too large", name);
    const int64_t rows = SW ? 2 * N : N;      // rows of one expert matrix
    if (nsb > (1 << 24) || rows > ((int64_t)1 << 40) / nsb) return fail(QMV_EINVAL, "%s: matrix too large", name);
    const int64_t mbytes = rows * nsb * Fmt::kBytes;
    if (estride < mbytes || estride % Fmt::kWAlign)
        return fail(QMV_EINVAL, "%s: expert_stride_bytes (%lld) must be >= %lld and a multiple of %d", name,
                    (long long)estride, (long long)mbytes, Fmt::kWAlign);
    if (E > 1 && estride > ((int64_t)1 << 46) / (E - 1)) return fail(QMV_EINVAL, "%s: experts too large", name);
    if (batch > 1 && xs_tok < K) return fail(QMV_EINVAL, "%s: x_stride_token must be >= n_cols", name);
    if (xs_tok < 0) return fail(QMV_EINVAL, "%s: x_stride_token must be >= 0", name);
    if (top_k > 1 && xs_slot != 0 && xs_slot < K)
        return fail(QMV_EINVAL, "%s: x_stride_slot must be 0 or >= n_cols", name);
    if (xs_slot < 0) return fail(QMV_EINVAL, "%s: x_stride_slot must be >= 0", name);
    if (!aligned(Wx, Fmt::kWAlign))
        return fail(QMV_EALIGN, "%s: W_experts must be %d-byte aligned for %s", name, Fmt::kWAlign, Fmt::kLabel);
    if (!aligned(y, 4) || !aligned(ids, 4))
        return fail(QMV_EALIGN, "%s: the output and expert_ids must be 4-byte aligned", name);
    if (!aligned(x, sizeof(XT))) return fail(QMV_EALIGN, "%s: x must be aligned to its %zu-byte elements", name,
                                             sizeof(XT));
    if (4 * nsb * kSbXPad * (int64_t)sizeof(float) > kLdsMax)
        return fail(QMV_EINVAL, "%s: n_cols %lld too large for one activation row in LDS", name, (long long)K);
    const SbRoute route{ids, estride, xs_tok, xs_slot, top_k, E};
    return sb_launch_lpr<Fmt, 1, XT, SW>(static_cast<const uint8_t*>(Wx), N, (int)nsb, x, K, y, N,
                                         as_stream(stream), &route, batch * top_k);
}

template <class Fmt, bool SW>
int32_t sb_moe_x(const char* name, const void* Wx, int64_t estride, int32_t E, int64_t N, int64_t K,
                 const int32_t* ids, int32_t batch, int32_t top_k, const void* x, int32_t x_type, int64_t xs_tok,
                 int64_t xs_slot, float* y, void* stream) {
    switch (x_type) {
    case QMV_X_F32:
        return sb_moe_t<Fmt, float, SW>(name, Wx, estride, E, N, K, ids, batch, top_k, static_cast<const float*>(x),
                                        xs_tok, xs_slot, y, stream);
    case QMV_X_F16:
        return sb_moe_t<Fmt, _Float16, SW>(name, Wx, estride, E, N, K, ids, batch, top_k,
                                           static_cast<const _Float16*>(x), xs_tok, xs_slot, y, stream);
    case QMV_X_BF16:
        return sb_moe_t<Fmt, __bf16, SW>(name, Wx, estride, E, N, K, ids, batch, top_k,
                                         static_cast<const __bf16*>(x), xs_tok, xs_slot, y, stream);
    default: return fail(QMV_EINVAL, "%s: unknown activation type %d", name, (int)x_type);
    }
}

template <class Fmt>
int32_t sb_moe(const char* name, bool swiglu, const void* Wx, int64_t estride, int32_t E, int64_t N, int64_t K,
               const int32_t* ids, int32_t batch, int32_t top_k, const void* x, int32_t x_type, int64_t xs_tok,
               int64_t xs_slot, float* y, void* stream) {
    if (swiglu) {
        if constexpr (Fmt::kSwiglu)
            return sb_moe_x<Fmt, true>(name, Wx, estride, E, N, K, ids, batch, top_k, x, x_type, xs_tok, xs_slot, y,
                                       stream);
        return fail(QMV_EUNSUPPORTED, "%s: the fused SwiGLU form is not offered for %s", name, Fmt::kLabel);
    }
    return sb_moe_x<Fmt, false>(name, Wx, estride, E, N, K, ids, batch, top_k, x, x_type, xs_tok, xs_slot, y, stream);
}

// MoE down with the router-weighted combine (formats whose table has a
// combine kernel): grid (row ranges, tokens), ranges x tokens filling the
// GPU once, a range holding at most kSbCombineRows rows; 8 waves per
// workgroup at batch 1..2 (about one row tile per workgroup: one wave per
// (slot, tile) unit of a token's 8 slots), else 4.
template <class Fmt, int LPR, int NW>
int32_t sb_combine_launch(const uint8_t* Wx, int64_t estride, int E, int64_t N, int nsb, const int32_t* ids,
                          const float* wts, int batch, int top_k, const float* x, int64_t xs_tok, int64_t xs_slot,
                          float* out, int xvec, hipStream_t st) {
    const char* name = "qmv_moe_combine";
    constexpr int RW = 64 / LPR;
    auto kern = Fmt::template combine_kernel<LPR, NW>();
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, name, &dyn_max)) return e;
    const size_t per_col = (size_t)4 * nsb * kSbXPad * sizeof(float);
    const size_t sums_max = (size_t)top_k * (kSbCombineRows + RW) * sizeof(float);
    if (per_col + sums_max > dyn_max)
        return fail(QMV_EINVAL, "%s: n_cols %d too large for one activation row in LDS", name, nsb * kSbWeights);
    const int SC = (int)std::min<size_t>((size_t)top_k, (dyn_max - sums_max) / per_col);
    const int64_t ntiles = (N + RW - 1) / RW;
    const int per_cu = std::max(1, resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW,
                                                SC * per_col + (size_t)top_k * NW * RW * sizeof(float)));
    const int64_t min_ranges = (ntiles * RW + kSbCombineRows - 1) / kSbCombineRows;
    const int64_t gx = std::max<int64_t>(
        min_ranges, std::min<int64_t>(ntiles, std::max<int64_t>(1, (int64_t)device_cu_count() * per_cu / batch)));
    const int64_t per_wg = (ntiles + gx - 1) / gx;
    const int rows_wg = (int)(per_wg * RW);
    const size_t lds = SC * per_col + (size_t)top_k * rows_wg * sizeof(float);
    hipLaunchKernelGGL(kern, dim3((unsigned)gx, (unsigned)batch), dim3(64 * NW), lds, st, Wx, estride, E, N, nsb,
                       ids, wts, top_k, x, xs_tok, xs_slot, out, xvec, SC, rows_wg);
    return check_launch(name);
}

template <class Fmt>
int32_t sb_combine(const void* Wx, int64_t estride, int32_t E, int64_t N, int64_t K, const int32_t* ids,
                   const float* wts, int32_t batch, int32_t top_k, const float* x, int64_t xs_tok, int64_t xs_slot,
                   float* out, void* stream) {
    const char* name = "qmv_moe_combine";
    if constexpr (!Fmt::kCombine) {
        return fail(QMV_EUNSUPPORTED, "%s: %s experts are not supported", name, Fmt::kLabel);
    } else {
        if (!Wx || !ids || !wts || !x || !out) return fail(QMV_EINVAL, "%s: null pointer", name);
        if (E < 1) return fail(QMV_EINVAL, "%s: n_experts must be >= 1", name);
        if (N < 1 || K < kSbWeights || K % kSbWeights)
            return fail(QMV_EINVAL, "%s: bad matrix shape %lld x %lld (n_cols a multiple of 256 for %s)", name,
                        (long long)N, (long long)K, Fmt::kLabel);
        if (batch < 1 || batch > 8) return fail(QMV_EINVAL, "%s: batch must be in 1..8 (got %d)", name, batch);
        if (top_k < 1 || top_k > kSbMaxSlots)
            return fail(QMV_EINVAL, "%s: top_k must be in 1..16 (got %d)", name, top_k);
        const int64_t nsb = K / kSbWeights;
        if (nsb > (1 << 24) || N > ((int64_t)1 << 40) / nsb) return fail(QMV_EINVAL, "%s: matrix too large", name);
        const int64_t mbytes = N * nsb * Fmt::kBytes;
        if (estride < mbytes || estride % Fmt::kWAlign)
            return fail(QMV_EINVAL, "%s: expert_stride_bytes (%lld) must be >= %lld and a multiple of %d", name,
                        (long long)estride, (long long)mbytes, Fmt::kWAlign);
        if (E > 1 && estride > ((int64_t)1 << 46) / (E - 1)) return fail(QMV_EINVAL, "%s: experts too large", name);
        if (batch > 1 && xs_tok < K) return fail(QMV_EINVAL, "%s: x_stride_token must be >= n_cols", name);
        if (xs_tok < 0) return fail(QMV_EINVAL, "%s: x_stride_token must be >= 0", name);
        if (top_k > 1 && xs_slot != 0 && xs_slot < K)
            return fail(QMV_EINVAL, "%s: x_stride_slot must be 0 or >= n_cols", name);
        if (xs_slot < 0) return fail(QMV_EINVAL, "%s: x_stride_slot must be >= 0", name);
        if (!aligned(Wx, Fmt::kWAlign))
            return fail(QMV_EALIGN, "%s: W_experts must be %d-byte aligned for %s", name, Fmt::kWAlign, Fmt::kLabel);
        if (!aligned(out, 4) || !aligned(ids, 4) || !aligned(wts, 4) || !aligned(x, 4))
            return fail(QMV_EALIGN, "%s: x, out, expert_ids and weights must be 4-byte aligned", name);
        const int xvec = (aligned(x, 16) && xs_tok % 4 == 0 && xs_slot % 4 == 0) ? 1 : 0;
        const uint8_t* W8 = static_cast<const uint8_t*>(Wx);
        hipStream_t st = as_stream(stream);
        auto go = [&](auto lpr) {
            constexpr int L = decltype(lpr)::value;
            return batch <= 2 ? sb_combine_launch<Fmt, L, 8>(W8, estride, E, N, (int)nsb, ids, wts, batch, top_k, x,
                                                             xs_tok, xs_slot, out, xvec, st)
                              : sb_combine_launch<Fmt, L, 4>(W8, estride, E, N, (int)nsb, ids, wts, batch, top_k, x,
                                                             xs_tok, xs_slot, out, xvec, st);
        };
        switch (sb_pick_lpr(4 * nsb)) {
        case 64: return go(std::integral_constant<int, 64>{});
        case 32: return go(std::integral_constant<int, 32>{});
        case 16: return go(std::integral_constant<int, 16>{});
        default: return go(std::integral_constant<int, 8>{});
        }
    }
}
// The chain-group slot of a super-block format's table (qmv_chain of these
// formats groups through sb_chain below).
inline bool sb_no_group(const RowSegs&, int, const float*, hipStream_t, bool, int32_t*) { return false; }

// Stages sharing one x as one launch over their concatenated rows
// (formats with a group kernel).
template <class Fmt, int LPR>
int32_t sb_group_launch(const RowSegs& segs, int nsb, const float* x, hipStream_t st) {
    constexpr int NW = 8;
    constexpr int RW = 64 / LPR;
    auto kern = Fmt::template group_kernel<LPR, NW>();
    const size_t lds = (size_t)4 * nsb * kSbXPad * sizeof(float);
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv_chain", &dyn_max)) return e;
    if (lds > dyn_max) return fail(QMV_EINVAL, "qmv_chain: %zu bytes of staged activations exceed the LDS", lds);
    const int64_t rows = segs.end[segs.n - 1];
    const int64_t tiles = (rows + NW * RW - 1) / (NW * RW);
    const int per_cu = std::max(1, resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds));
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, (int64_t)device_cu_count() * per_cu));
    const int xvec = aligned(x, 16) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, segs, nsb, x, xvec);
    return check_launch("qmv_chain");
}

// qmv_chain for a super-block format: stages in order, each run of up to
// kMaxSegs stages that read one x with one width and do not wait as one
// launch over their concatenated rows (formats with a group kernel), every
// other stage as the batch-1 entry point's launch.  Stream order stands in
// for the stage barriers, so no workspace is used; each output is bitwise
// the batch-1 entry point's.
template <class Fmt>
int32_t sb_chain(const char* name, const qmv_chain_stage* stages, int32_t n_stages, void* stream) {
    if (!stages) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (n_stages < 1) return fail(QMV_EINVAL, "%s: n_stages must be >= 1", name);
    for (int s = 0; s < n_stages; ++s) {
        const qmv_chain_stage& q = stages[s];
        if (!q.W || !q.x || !q.y) return fail(QMV_EINVAL, "%s: stage %d: null pointer", name, s);
        if (q.n_rows < 1 || q.n_rows > (1 << 30))
            return fail(QMV_EINVAL, "%s: stage %d: n_rows must be in 1..2^30", name, s);
        if (q.n_cols < kSbWeights || q.n_cols % kSbWeights || 4 * (q.n_cols / kSbWeights) * kSbXPad * 4 > kLdsMax)
            return fail(QMV_EINVAL, "%s: stage %d: n_cols must be a multiple of 256 in 256..38400 for %s", name, s,
                        Fmt::kLabel);
        if (!aligned(q.W, Fmt::kWAlign))
            return fail(QMV_EALIGN, "%s: stage %d: W must be %d-byte aligned for %s", name, s, Fmt::kWAlign,
                        Fmt::kLabel);
        if (!aligned(q.x, 4) || !aligned(q.y, 4))
            return fail(QMV_EALIGN, "%s: stage %d: x and y must be 4-byte aligned", name, s);
    }
    hipStream_t st = as_stream(stream);
    for (int i = 0; i < n_stages;) {
        const qmv_chain_stage& q = stages[i];
        const int nsb = (int)(q.n_cols / kSbWeights);
        int j = i + 1;
        while (j < n_stages && j - i < kMaxSegs && !stages[j].wait && stages[j].x == q.x &&
               stages[j].n_cols == q.n_cols)
            ++j;
        int32_t rc = QMV_OK;
        if constexpr (Fmt::kGroup) {
            if (j - i > 1) {
                RowSegs segs = {};
                segs.n = j - i;
                int64_t rows = 0;
                for (int k = i; k < j; ++k) {
                    segs.W[k - i] = static_cast<const uint8_t*>(stages[k].W);
                    segs.y[k - i] = stages[k].y;
                    rows += stages[k].n_rows;
                    segs.end[k - i] = rows;
                }
                switch (sb_pick_lpr(4 * nsb)) {
                case 64: rc = sb_group_launch<Fmt, 64>(segs, nsb, q.x, st); break;
                case 32: rc = sb_group_launch<Fmt, 32>(segs, nsb, q.x, st); break;
                case 16: rc = sb_group_launch<Fmt, 16>(segs, nsb, q.x, st); break;
                default: rc = sb_group_launch<Fmt, 8>(segs, nsb, q.x, st); break;
                }
                if (rc != QMV_OK) return rc;
                i = j;
                continue;
            }
        }
        for (int k = i; k < j; ++k) {
            const qmv_chain_stage& r = stages[k];
            rc = sb_launch_lpr<Fmt, 1, float>(static_cast<const uint8_t*>(r.W), r.n_rows, nsb, r.x, r.n_cols, r.y,
                                              r.n_rows, st);
            if (rc != QMV_OK) return rc;
        }
        i = j;
    }
    return ok();
}

template <class Fmt>
const FormatOps& sb_format_ops() {
    static const FormatOps ops = {sb_matvec<Fmt>, sb_dequant<Fmt>, sb_moe<Fmt>, sb_combine<Fmt>, sb_no_group,
                                  sb_chain<Fmt>};
    return ops;
}

}  // namespace
}  // namespace qmv
