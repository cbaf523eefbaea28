// Block-quantized (Q8_0 / Q4_0 / Q4_1) matrix x vector kernels for gfx950:
// the kernels and launchers, templated on the format.  Each format's
// instantiations are compiled in a translation unit of their own
// (qmv_fmt_q8_0.hip, qmv_fmt_q4_0.hip, qmv_fmt_q4_1.hip), which exports them
// as a FormatOps table; qmv_blocks.hip holds the C entry points.
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
//  * The activation vector is the only thing staged in LDS in this kernel:
//    x[b] once per workgroup, padded to 36 floats per 32-block so that the
//    16-byte LDS reads of neighbouring lanes fall in different banks.
//  * Each lane accumulates RPL rows x B columns in fp32; a segment then
//    reduces across its LPR lanes with cross-lane shuffles in a fixed order
//    (deterministic, no atomics).
//  * No MFMA: at batch 1..8 this is a GEMV, bound by HBM bandwidth.
#pragma once
#include <cmath>
#include <type_traits>

#include "qmv_block_decode.h"

namespace qmv {
namespace {

// ------------------------------------------------------------------ kernels
// Routing of the dense kernel (ROUTE = true): grid row p = b * top_k + s
// (blockIdx.y) computes the pair (token b, slot s), with expert ids[p]
// (weights at ids[p] * estride), activations at b * xs_tok + s * xs_slot
// and outputs at p * ldy.  An id outside [0, n_experts) makes that pair's
// outputs quiet NaN.
struct PairRoute {
    const int32_t* ids;
    int64_t estride;
    int64_t xs_tok, xs_slot;
    int32_t top_k, n_experts;
};

// Dense matvec.  A persistent grid (as many workgroups as fit on the GPU at
// once); wave w of the grid takes row tiles w, w + waves, ... .  A tile is
// G*RPL rows (G row segments of LPR lanes, RPL rows per lane) and is worked
// through in T = ceil(nb/LPR) steps; in step t lane li reads block
// li + LPR*t of each of its RPL rows.  The blocks of the next step are
// loaded while the current step is computed (two steps in flight per wave),
// and the first step's loads are issued before the activation staging so
// that both latencies overlap.  SWG (routed, RPL = 2): the expert holds 2N
// rows, gate rows then up rows; output row i pairs gate row i with up row
// N + i in the same lanes and writes SiLU(gate) * up.
template <class F, int B, int LPR, int RPL, int XU, int NW, int PD = 2, bool ROUTE = false, class XT = float,
          bool SWG = false>
__global__ __launch_bounds__(64 * NW) void qmv_kernel(const uint8_t* __restrict__ W, int64_t N, int nb,
                                                       const XT* __restrict__ x, int64_t ldx,
                                                       float* __restrict__ y, int64_t ldy, int xvec,
                                                       const PairRoute route) {
    static_assert(!SWG || (RPL == 2 && B == 1), "paired gate/up rows: two rows per lane, one column");
    extern __shared__ __attribute__((aligned(16))) float lds[];   // 16-byte aligned after any static LDS
    float* xs = lds;

    constexpr int G = 64 / LPR;
    constexpr int ROWS = SWG ? G : G * RPL;   // output rows per tile
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int T = (nb + LPR - 1) / LPR;
    const int64_t ntiles = (N + ROWS - 1) / ROWS;
    const int64_t wstride = (int64_t)gridDim.x * NW;
    bool bad = false;   // routed pair with an invalid id: outputs become NaN
    if constexpr (ROUTE) {
        // No branch: an invalid id streams expert 0 (valid memory) and its
        // outputs are replaced, so the prologue below stays straight-line.
        const int p = blockIdx.y;
        const int e = route.ids[p];          // uniform: one scalar load
        bad = e < 0 || e >= route.n_experts;
        W += (int64_t)(bad ? 0 : e) * route.estride;
        x += (int64_t)(p / route.top_k) * route.xs_tok + (int64_t)(p % route.top_k) * route.xs_slot;
        y += (int64_t)p * ldy;
    }

    // Step (tile, t): lane li handles block li + LPR*t of its RPL rows.
    using Raw = typename F::Raw;
    auto load_step = [&](int64_t tile, int t, Raw (&blk)[RPL]) {
        const int j = min(li + LPR * t, nb - 1);      // clamp: stays in bounds
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int64_t row = SWG ? min(tile * G + seg, N - 1) + r * N : min(tile * ROWS + r * G + seg, N - 1);
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
        float d[RPL], m[RPL];
        uint32_t c[RPL][8];
#pragma unroll
        for (int r = 0; r < RPL; ++r) F::decode(blk[r], d[r], m[r], c[r]);
        float sdot[RPL][B];
        dot_multi<F, RPL, B>(c, d, m, xj, nb * kXPad, sdot, B);
#pragma unroll
        for (int r = 0; r < RPL; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float upd = Term<F>::add(acc[r][b], d[r], m[r], sdot[r][b]);
                acc[r][b] = valid ? upd : acc[r][b];
            }
        if (t == T - 1) {   // tile done: reduce the segments and write
#pragma unroll
            for (int r = 0; r < RPL; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) acc[r][b] = segment_sum<LPR>(acc[r][b]);
            if (li == 0) {
                if constexpr (SWG) {
                    const int64_t row = tile * G + seg;
                    if (row < N) y[row] = bad ? __builtin_nanf("") : silu(acc[0][0]) * acc[1][0];
                } else {
#pragma unroll
                    for (int r = 0; r < RPL; ++r) {
                        const int64_t row = tile * ROWS + r * G + seg;
                        if (row < N) {
#pragma unroll
                            for (int b = 0; b < B; ++b) y[b * ldy + row] = bad ? __builtin_nanf("") : acc[r][b];
                        }
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

    // Two register buffers used in turn: while one step is computed the
    // loads of the next are in flight.  Once the load cursor is past the
    // wave's last step, the step in hand is the last one: it is computed
    // after the loop and nothing more is loaded.  (A wave without any step
    // loads the last tile's first step once, clamped in bounds, unused.)
    Raw buf[PD][RPL];
    int64_t ltile = (int64_t)blockIdx.x * NW + wave;   // next step to load
    int lt = 0;
    int64_t ctile = ltile;                             // next step to compute
    int ct = 0;
    const int K4 = nb * 8;
    auto load_next = [&](Raw (&b)[RPL]) {
        load_step(min(ltile, ntiles - 1), ltile < ntiles ? lt : 0, b);
        if (ltile < ntiles) advance(ltile, lt);
    };
    if (XU > 0 && xvec) {
        // batch 1: x loads, then the first weight loads, then x into LDS
        XStage<XU, 64 * NW, XT> xst;
        xst.load(x, K4);
#pragma unroll
        for (int p = 0; p < PD - 1; ++p) load_next(buf[p]);
        __builtin_amdgcn_sched_barrier(0);   // keep both batches of loads issued first
        xst.store(xs, K4);
        __syncthreads();
    } else {
        const XT* xcol[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xcol[b] = x + b * ldx;
        stage_x_cols<B, 64 * NW, XT>(xcol, nb, xs, B, xvec != 0);
#pragma unroll
        for (int p = 0; p < PD - 1; ++p) load_next(buf[p]);
    }

    static_assert(PD == 2, "pipeline depth");
    if (ctile < ntiles) {
        while (ltile < ntiles) {
            load_next(buf[1]);
            __builtin_amdgcn_sched_barrier(0);   // loads before using buf[0]
            compute_step(ctile, ct, buf[0]);
            advance(ctile, ct);
            if (ltile >= ntiles) {   // the last step is in buf[1]: one drain site below
#pragma unroll
                for (int r = 0; r < RPL; ++r) buf[0][r] = buf[1][r];
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

// Batch 1, rows of whole 64-block steps (nb % 64 == 0), W 16-byte aligned:
// the same lane-to-block mapping, arithmetic and reduction order as
// qmv_kernel<F, 1, 64, 1, ...> (bitwise the same y), but each step's 64
// blocks arrive as whole 16-byte chunks with non-temporal loads and are
// re-read block-aligned from a per-wave LDS scratch.  A wave works on RR
// rows at a time (rows RR*p .. RR*p + RR - 1 for p = wave, wave + grid
// waves, ...), so a step moves RR * 64 blocks.  The rows are those of up to
// kMaxSegs matrices sharing x, concatenated (a wave-uniform lookup finds a
// row's matrix).
template <class F, int XU, int NW, int PD = 2, class XT = float, int RR = 1>
__global__ __launch_bounds__(64 * NW) void qmv_kernel_c(const RowSegs segs, int nb, const XT* __restrict__ x) {
    using C = Contig<F>;
    extern __shared__ __attribute__((aligned(16))) float lds[];   // 16-byte aligned after any static LDS
    float* xs = lds;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint8_t* scratch = reinterpret_cast<uint8_t*>(lds + nb * kXPad) + wave * RR * C::kStepBytes;
    const int T = nb / 64;
    const int64_t wstride = (int64_t)gridDim.x * NW;
    // rows < 2^31 (checked by the launcher): 32-bit row arithmetic is scalar
    const int N = (int)segs.end[segs.n - 1];
    const int NP = (N + RR - 1) / RR;               // row groups
    const int wstride32 = (int)wstride;
    const uint32_t pitch = (uint32_t)nb * F::kBytes;  // bytes per row (< 2^32, checked)

    typename C::Chunks buf[PD][RR];
    int lrow = (int)blockIdx.x * NW + wave;          // next step to load (row group)
    int lt = 0;
    int crow = lrow;                                 // next step to compute
    int ct = 0;
    auto advance = [&](int& row, int& t) {
        if (++t == T) { t = 0; row += wstride32; }
    };
    // The matrix of a (wave-uniform) row: selects over the table with
    // constant indices only, so the table stays in scalar registers and the
    // lookup issues no dependent loads from the argument segment.
    auto locate = [&](int row, const uint8_t*& Wm, float*& ym, int& start) {
        Wm = segs.W[0];
        ym = segs.y[0];
        start = 0;
#pragma unroll
        for (int i = 1; i < kMaxSegs; ++i) {
            const bool in = i < segs.n && row >= (int)segs.end[i - 1];
            Wm = in ? segs.W[i] : Wm;
            ym = in ? segs.y[i] : ym;
            start = in ? (int)segs.end[i - 1] : start;
        }
    };
    // The load cursor keeps a buffer descriptor over each row of its row
    // group (wave-uniform, in scalar registers), set once per row group; a
    // step's loads are the descriptor, a scalar step offset and a per-lane
    // constant offset.
    __amdgpu_buffer_rsrc_t lrs[RR];
    int voff[C::kLoads];
    C::lane_offsets(lane, voff);
    auto set_rows = [&](int p) {
#pragma unroll
        for (int k = 0; k < RR; ++k) {
            const int row = min(RR * p + k, N - 1);
            const uint8_t* Wm;
            float* ym;
            int start;
            locate(row, Wm, ym, start);
            lrs[k] = raw_buffer(Wm + (int64_t)(row - start) * pitch, pitch);
        }
    };
    set_rows(min(lrow, NP - 1));
    // Called while the load cursor is inside the wave's rows, and once at
    // the start by waves without rows (clamped to the last row group).
    auto load_next = [&](typename C::Chunks (&c)[RR]) {
        const int soff = (lrow < NP ? lt : 0) * C::kStepBytes;
#pragma unroll
        for (int k = 0; k < RR; ++k) C::fetch(lrs[k], soff, voff, c[k]);
        if (lrow < NP && ++lt == T) {
            lt = 0;
            lrow += wstride32;
            set_rows(min(lrow, NP - 1));
        }
    };
    float acc[RR];
#pragma unroll
    for (int k = 0; k < RR; ++k) acc[k] = 0.f;
    auto compute_step = [&](int t, const typename C::Chunks (&c)[RR]) {
        const int j = lane + 64 * t;
        float d[RR], m[RR];
        uint32_t cd[RR][8];
#pragma unroll
        for (int k = 0; k < RR; ++k) {
            typename F::Raw r;
            C::to_block(c[k], scratch + k * C::kStepBytes, lane, r);
            F::decode(r, d[k], m[k], cd[k]);
        }
        float sdot[RR][1];
        dot_multi<F, RR, 1>(cd, d, m, xs + j * kXPad, nb * kXPad, sdot, 1);
#pragma unroll
        for (int k = 0; k < RR; ++k) acc[k] = Term<F>::add(acc[k], d[k], m[k], sdot[k][0]);
        if (t == T - 1) {
#pragma unroll
            for (int k = 0; k < RR; ++k) {
                const float tot = segment_sum<64>(acc[k]);
                const int row = RR * crow + k;
                if (row < N) {
                    const uint8_t* Wm;
                    float* ym;
                    int start;
                    locate(row, Wm, ym, start);
                    if (lane == 0) ym[row - start] = tot;
                }
                acc[k] = 0.f;
            }
        }
    };

    const int K4 = nb * 8;
    if (XU > 0) {
        XStage<XU, 64 * NW, XT> xst;
        xst.load(x, K4);
#pragma unroll
        for (int p = 0; p < PD - 1; ++p) load_next(buf[p]);
        __builtin_amdgcn_sched_barrier(0);
        xst.store(xs, K4);
        __syncthreads();
    } else {
        const XT* xcol[1] = {x};
        stage_x_cols<1, 64 * NW, XT>(xcol, nb, xs, 1, true);
#pragma unroll
        for (int p = 0; p < PD - 1; ++p) load_next(buf[p]);
    }

    // The load cursor runs one step ahead; once it is past the wave's last
    // step, the step in hand is the last one and nothing more is loaded (no
    // loads past the end: with every idle wave re-reading one place they
    // queued on a few L2 channels).
    static_assert(PD == 2, "pipeline depth");
    static_assert(RR == 1 || RR == 2, "rows per step");
    if (crow < NP) {
        while (lrow < NP) {
            load_next(buf[1]);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(ct, buf[0]);
            advance(crow, ct);
            if (lrow >= NP) {   // the last step is in buf[1]: one drain site below
#pragma unroll
                for (int k = 0; k < RR; ++k) buf[0][k] = buf[1][k];
                break;
            }
            load_next(buf[0]);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(ct, buf[1]);
            advance(crow, ct);
        }
        compute_step(ct, buf[0]);
    }
}

// Grouped MoE expert matvec.  blockIdx.y = u selects the u-th distinct
// expert id in first-occurrence order of ids[0..P); the workgroup streams
// rows [blockIdx.x*ROWS_WG, +ROWS_WG) of that expert once per group of up
// to 8 (token, slot) pairs routed to it (one group in the usual case of
// distinct ids per token), in pair order.
constexpr int kMoeMaxPairs = 128;
constexpr int kMoeMaxSlots = 16;     // top_k
constexpr int kMoeStaticLds = 4096;  // s_ids/s_first/s_members/scalars, rounded up

// One chunk of up to BC member pairs of expert We: stage their activations
// and stream the workgroup's row tiles [tb, te) once.  A row tile holds G
// output rows; output row i reads matrix row i, and with RS = 2 also row
// N + i (the up row paired with gate row i of a row-concatenated gate||up
// expert).  When a row is done, emit(b, row, t0, t1) receives member b's
// sums of the row (t1: of row N + row when RS = 2) in the row's first lane.
// XU > 0 (the activations fit in XU 16-byte loads per thread and are
// 16-byte aligned): the activation loads are issued first, then the first
// weight loads, and only then are the activations stored to LDS, so the two
// latencies overlap (loads complete in order).  XU == 0: staged by the
// looping stager, then the weights.  Ends with a barrier.
template <class F, int BC, int LPR, int NW, int XU, int PD, int RS, class XT, class Emit>
__device__ __forceinline__ void moe_chunk(const uint8_t* __restrict__ We, int64_t N, int nb, int64_t tb, int64_t te,
                                          const XT* const (&xcol)[BC], int w, bool xvec, float* xs, Emit&& emit) {
    constexpr int G = 64 / LPR;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int T = (nb + LPR - 1) / LPR;
    using Raw = typename F::Raw;
    int64_t ltile = tb + wave, ctile = ltile;
    int lt = 0, ct = 0;
    auto advance = [&](int64_t& tile, int& st) {
        if (++st == T) { st = 0; tile += NW; }
    };
    auto load_next = [&](Raw (&r)[RS]) {
        const int64_t tile = min(ltile, te - 1);       // past the range (prologue only): a block in range
        const int j = min(li + LPR * (ltile < te ? lt : 0), nb - 1);
        const int64_t row = min(tile * G + seg, N - 1);
#pragma unroll
        for (int k = 0; k < RS; ++k) F::fetch(We, (row + k * N) * nb + j, r[k]);
        if (ltile < te) advance(ltile, lt);
    };
    float acc[RS][BC];
#pragma unroll
    for (int k = 0; k < RS; ++k)
#pragma unroll
        for (int b = 0; b < BC; ++b) acc[k][b] = 0.f;
    auto compute_step = [&](int64_t tile, int st, const Raw (&r)[RS]) {
        const int j = li + LPR * st;
        const bool valid = j < nb;
        const int jc = valid ? j : nb - 1;
        float d[RS], m[RS];
        uint32_t c[RS][8];
#pragma unroll
        for (int k = 0; k < RS; ++k) F::decode(r[k], d[k], m[k], c[k]);
        float s[RS][BC];
        dot_multi<F, RS, BC>(c, d, m, xs + jc * kXPad, nb * kXPad, s, w);
#pragma unroll
        for (int b = 0; b < BC; ++b) {
            if (b < w) {
#pragma unroll
                for (int k = 0; k < RS; ++k) {
                    const float upd = Term<F>::add(acc[k][b], d[k], m[k], s[k][b]);
                    acc[k][b] = valid ? upd : acc[k][b];
                }
            }
        }
        if (st == T - 1) {
            const int64_t row = tile * G + seg;
#pragma unroll
            for (int b = 0; b < BC; ++b) {
                if (b < w) {
                    const float t0 = segment_sum<LPR>(acc[0][b]);
                    const float t1 = RS > 1 ? segment_sum<LPR>(acc[RS - 1][b]) : 0.f;
                    if (li == 0 && row < N) emit(b, row, t0, t1);
                }
#pragma unroll
                for (int k = 0; k < RS; ++k) acc[k][b] = 0.f;
            }
        }
    };

    Raw buf[PD][RS];
    const int K4 = nb * 8;
    if constexpr (XU > 0) {
        // every column slot is loaded and stored (inactive ones repeat
        // column 0): straight-line code, so no branch merges the waits
        XStage<XU, 64 * NW, XT> xst[BC];
#pragma unroll
        for (int b = 0; b < BC; ++b) xst[b].load(xcol[b], K4);
#pragma unroll
        for (int p = 0; p < PD - 1; ++p) load_next(buf[p]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < BC; ++b) xst[b].store(xs + b * nb * kXPad, K4);
        __syncthreads();
    } else {
        stage_x_cols<BC, 64 * NW, XT>(xcol, nb, xs, w, xvec);
#pragma unroll
        for (int p = 0; p < PD - 1; ++p) load_next(buf[p]);
    }

    // The load cursor runs PD - 1 steps ahead.  Once it is past the range,
    // the steps still in flight (buffer P first, then the next) are moved to
    // buf[0], buf[1] in order and computed at one site after the loop, so no
    // load goes past the wave's last step (idle re-reads of one place queued
    // on a few L2 channels).
    static_assert(PD == 2 || PD == 3, "pipeline depth");
    auto rotate_to_front = [&](int P) {
        if (PD == 2) {
            if (P == 1)
#pragma unroll
                for (int k = 0; k < RS; ++k) buf[0][k] = buf[1][k];
        } else if (P == 1) {
#pragma unroll
            for (int k = 0; k < RS; ++k) {
                buf[0][k] = buf[1][k];
                buf[1][k] = buf[PD - 1][k];
            }
        } else if (P == 2) {
#pragma unroll
            for (int k = 0; k < RS; ++k) {
                const Raw tmp = buf[0][k];
                buf[0][k] = buf[PD - 1][k];
                buf[1][k] = tmp;
            }
        }
    };
#define QMV_MOE_STEP(P)                                    \
    {                                                      \
        if (ltile >= te) {                                 \
            rotate_to_front(P);                            \
            break;                                         \
        }                                                  \
        load_next(buf[((P) + PD - 1) % PD]);               \
        __builtin_amdgcn_sched_barrier(0);                 \
        compute_step(ctile, ct, buf[(P)]);                 \
        advance(ctile, ct);                                \
    }
    if (ctile < te) {
        while (true) {
            QMV_MOE_STEP(0)
            QMV_MOE_STEP(1)
            if constexpr (PD >= 3) QMV_MOE_STEP(2)
        }
#pragma unroll 1
        for (int i = 0; i < PD - 1 && ctile < te; ++i) {
            compute_step(ctile, ct, buf[0]);
            advance(ctile, ct);
            if (PD > 2)
#pragma unroll
                for (int k = 0; k < RS; ++k) buf[0][k] = buf[1][k];
        }
    }
#undef QMV_MOE_STEP
    __syncthreads();   // xs is restaged by the next chunk
}

// Grouped expert matvec.  Workgroup (bx, u) serves the u-th distinct id
// of the (token, slot) pairs, in first-occurrence order, and the bx-th
// range of that expert's row tiles: it groups the pairs itself (O(P) per
// thread for P <= 128 pairs; no prologue kernel, no workspace), then runs
// moe_chunk for up to BC member pairs at a time.  Per (row, pair) the
// arithmetic is the dense kernel's, so each output equals a single-expert
// dense call bitwise.  SW (SwiGLU): every expert holds 2N rows, gate rows
// then up rows, and output row i is SiLU(gate_i x) * (up_i x), both sums
// again the dense kernel's.
template <class F, int BC, int LPR, int NW, int XU, int PD, bool SW = false, class XT = float>
__global__ __launch_bounds__(64 * NW) void moe_kernel(const uint8_t* __restrict__ Wx, int64_t estride,
                                                       int n_experts, int64_t N, int nb,
                                                       const int32_t* __restrict__ ids, int P, int top_k,
                                                       const XT* __restrict__ x, int64_t xs_tok,
                                                       int64_t xs_slot, float* __restrict__ y, int xvec) {
    static_assert(64 * NW >= kMoeMaxPairs, "one thread per pair");
    __shared__ int s_ids[kMoeMaxPairs];
    __shared__ int s_first[kMoeMaxPairs];
    __shared__ int s_members[kMoeMaxPairs];
    __shared__ int s_expert, s_has, s_nmem;
    extern __shared__ __attribute__((aligned(16))) float lds[];   // 16-byte aligned after any static LDS
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

    constexpr int G = 64 / LPR;
    const int64_t ntiles = (N + G - 1) / G;
    const int64_t per_wg = (ntiles + gridDim.x - 1) / gridDim.x;
    const int64_t tb = (int64_t)blockIdx.x * per_wg;
    const int64_t te = min(ntiles, tb + per_wg);
    if (tb >= te) return;
    if (e < 0 || e >= n_experts) {
        // An id outside [0, n_experts) cannot be reported to the host:
        // its outputs become quiet NaN.
        const float qnan = __builtin_nanf("");
        for (int k = 0; k < nmem; ++k)
            for (int64_t row = tb * G + t; row < te * G && row < N; row += 64 * NW)
                y[(int64_t)s_members[k] * N + row] = qnan;
        return;
    }
    const uint8_t* __restrict__ We = Wx + (int64_t)e * estride;
    float* xs = lds;
    for (int c0 = 0; c0 < nmem; c0 += BC) {
        const int w = min(BC, nmem - c0);
        const XT* xcol[BC];
#pragma unroll
        for (int b = 0; b < BC; ++b) {
            const int pr = s_members[c0 + (b < w ? b : 0)];
            xcol[b] = x + (int64_t)(pr / top_k) * xs_tok + (int64_t)(pr % top_k) * xs_slot;
        }
        const int* mem = s_members + c0;
        auto emit = [&](int b, int64_t row, float t0, float t1) {
            y[(int64_t)mem[b] * N + row] = SW ? silu(t0) * t1 : t0;
        };
        constexpr int RS = SW ? 2 : 1;
        if (c0 == 0 && XU > 0 && xvec)
            moe_chunk<F, BC, LPR, NW, XU, PD, RS, XT>(We, N, nb, tb, te, xcol, w, true, xs, emit);
        else
            moe_chunk<F, BC, LPR, NW, 0, PD, RS, XT>(We, N, nb, tb, te, xcol, w, xvec != 0, xs, emit);
    }
}

// MoE down projection with the router-weighted combine, token-major:
// workgroup (bx, b) computes rows of out[b] = sum_s w[b][s] * DEQ(W_{e_s}) x_{b,s}
// over the top_k slots of token b.  The slots' activation vectors are
// staged together (in chunks of SC slots when they do not all fit the LDS).
// The work is the units (slot, row tile); wave w takes units w, w + NW,
// ... with one pipeline running across them, and each unit's row sums (the
// dense kernel's, bitwise the qmv_moe outputs) go to LDS.  Then one thread
// per row adds them in slot order: fma(w_s, y_s, acc) from s = 0 up.  Every
// (token, slot) streams its expert: experts shared by several tokens are
// read once per token, which is what keeps the combine free of atomics and
// workspace.
template <class F, int LPR, int NW, int PD>
__global__ __launch_bounds__(64 * NW) void moe_combine_kernel(const uint8_t* __restrict__ Wx, int64_t estride,
                                                               int n_experts, int64_t N, int nb,
                                                               const int32_t* __restrict__ ids,
                                                               const float* __restrict__ wts, int top_k,
                                                               const float* __restrict__ x, int64_t xs_tok,
                                                               int64_t xs_slot, float* __restrict__ out, int xvec,
                                                               int SC, int rows_wg) {
    __shared__ const uint8_t* s_base[kMoeMaxSlots];
    __shared__ float s_w[kMoeMaxSlots];
    __shared__ int s_bad;
    extern __shared__ __attribute__((aligned(16))) float lds[];   // 16-byte aligned after the static LDS
    constexpr int G = 64 / LPR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int seg = lane / LPR, li = lane % LPR;
    const int T = (nb + LPR - 1) / LPR;
    const int b = blockIdx.y;
    const int64_t ntiles = (N + G - 1) / G;
    const int per_wg = rows_wg / G;
    const int64_t tb = (int64_t)blockIdx.x * per_wg;
    const int64_t te = min(ntiles, tb + per_wg);
    if (tb >= te) return;
    const int wtiles = (int)(te - tb);
    const int per_col = nb * kXPad;
    float* xs = lds;                          // [SC][nb][kXPad]
    float* ybuf = lds + SC * per_col;         // [top_k][rows_wg]: row sums per slot
    const int64_t r0 = tb * G;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    if (tid < top_k) {
        const int e = ids[b * top_k + tid];
        const bool eb = e < 0 || e >= n_experts;
        if (eb) s_bad = 1;
        s_base[tid] = Wx + (int64_t)(eb ? 0 : e) * estride;
        s_w[tid] = wts[b * top_k + tid];
    }
    using Raw = typename F::Raw;
    __syncthreads();   // s_base, s_w
    for (int s0 = 0; s0 < top_k; s0 += SC) {
        const int sc = min(SC, top_k - s0);
        // this wave's units q = wave, wave + NW, ... of the chunk's
        // sc * wtiles (slot-major), T steps each
        const int units = sc * wtiles;
        const int my_units = wave < units ? (units - wave + NW - 1) / NW : 0;
        const int64_t nsteps = (int64_t)my_units * T;
        struct Cur {
            int q, t;
        };
        Cur lc{wave, 0}, cc = lc;
        auto advance = [&](Cur& k) {
            if (++k.t == T) {
                k.t = 0;
                k.q += NW;
            }
        };
        int64_t lrem = nsteps;
        int lslot = min(lc.q, units - 1) / wtiles;
        const uint8_t* lW = s_base[s0 + lslot];
        auto load_next = [&](Raw& r) {
            const int q = min(lc.q, units - 1);            // a wave without units re-reads a valid block
            const int slot = q / wtiles;
            const int64_t tile = tb + (q - slot * wtiles);
            const int64_t row = min(tile * G + seg, N - 1);
            const int j = min(li + LPR * lc.t, nb - 1);
            F::fetch(lW, row * nb + j, r);
            if (lrem > 1) {   // past the last step: re-read it (in cache)
                --lrem;
                advance(lc);
                const int ns = lc.q / wtiles;
                if (ns != lslot) {
                    lslot = ns;
                    lW = s_base[s0 + ns];
                }
            }
        };
        // the first weight loads go out before the activations are staged
        Raw buf[PD];
#pragma unroll
        for (int p = 0; p < PD - 1; ++p) load_next(buf[p]);
        // the chunk's activation vectors (every wave is done with the
        // previous chunk's: its units all ended before this barrier)
        __syncthreads();
        {
            // chunk i of the sc concatenated vectors, four loads in flight per thread
            const float* xb = x + (int64_t)b * xs_tok + (int64_t)s0 * xs_slot;
            const int per = xvec ? nb * 8 : nb * 32;          // float4 chunks or floats per vector
            const int total = sc * per;
            for (int i0 = tid; i0 < total; i0 += 4 * 64 * NW) {
                int k4[4], c4[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = min(i0 + u * 64 * NW, total - 1);
                    k4[u] = i / per;
                    c4[u] = i - k4[u] * per;
                }
                if (xvec) {
                    float4 v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        v[u] = *reinterpret_cast<const float4*>(xb + (int64_t)k4[u] * xs_slot + 4 * c4[u]);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int e = 4 * c4[u];
                        if (i0 + u * 64 * NW < total)
                            *reinterpret_cast<float4*>(xs + k4[u] * nb * kXPad + (e >> 5) * kXPad + (e & 31)) = v[u];
                    }
                } else {
                    float v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) v[u] = xb[(int64_t)k4[u] * xs_slot + c4[u]];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int e = c4[u];
                        if (i0 + u * 64 * NW < total) xs[k4[u] * nb * kXPad + (e >> 5) * kXPad + (e & 31)] = v[u];
                    }
                }
            }
        }
        __syncthreads();
        if (nsteps == 0) continue;
        float acc = 0.f;
        auto compute = [&](const Raw& r) {
            const int slot = cc.q / wtiles;
            const int64_t tile = tb + (cc.q - slot * wtiles);
            const int j = li + LPR * cc.t;
            const bool valid = j < nb;
            const int jc = valid ? j : nb - 1;
            float d, m;
            uint32_t c[1][8];
            F::decode(r, d, m, c[0]);
            float sd[1][1];
            const float dd[1] = {d}, mm[1] = {m};
            dot_multi<F, 1, 1>(c, dd, mm, xs + slot * nb * kXPad + jc * kXPad, 0, sd, 1);
            const float upd = Term<F>::add(acc, d, m, sd[0][0]);
            acc = valid ? upd : acc;
            if (cc.t == T - 1) {
                const float tot = segment_sum<LPR>(acc);
                const int64_t row = tile * G + seg;
                if (li == 0 && row < N) ybuf[(s0 + slot) * rows_wg + (row - r0)] = tot;
                acc = 0.f;
            }
        };
        int64_t crem = nsteps;
#define QMV_MOEC_STEP(P)                                   \
    {                                                      \
        load_next(buf[((P) + PD - 1) % PD]);               \
        __builtin_amdgcn_sched_barrier(0);                 \
        compute(buf[(P)]);                                 \
        if (--crem == 0) break;                            \
        advance(cc);                                       \
    }
        static_assert(PD >= 2 && PD <= 4, "pipeline depth");
        while (true) {
            QMV_MOEC_STEP(0)
            QMV_MOEC_STEP(1)
            if constexpr (PD >= 3) QMV_MOEC_STEP(2)
            if constexpr (PD >= 4) QMV_MOEC_STEP(3)
        }
#undef QMV_MOEC_STEP
    }
    __syncthreads();
    const float qnan = __builtin_nanf("");
    const int64_t r1 = min(te * G, N);
    for (int64_t row = r0 + tid; row < r1; row += 64 * NW) {
        const float* yr = ybuf + (row - r0);
        float v = s_w[0] * yr[0];
        for (int s = 1; s < top_k; ++s) v = __builtin_fmaf(s_w[s], yr[s * rows_wg], v);
        out[(int64_t)b * N + row] = s_bad ? qnan : v;
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

template <class F, int B, int LPR, int XU, int NW, class XT = float, int RPL = 1>
int32_t launch_b(const uint8_t* W, int64_t N, int nb, const XT* x, int64_t ldx, float* y, int64_t ldy,
                 hipStream_t st) {
    auto kern = qmv_kernel<F, B, LPR, RPL, XU, NW, 2, false, XT>;
    const size_t lds = (size_t)B * nb * kXPad * sizeof(float);
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv", &dyn_max)) return e;
    if (lds > dyn_max) return fail(QMV_EINVAL, "qmv: %zu bytes of staged activations exceed the LDS", lds);
    constexpr int rows_per_wg = NW * (64 / LPR) * RPL;
    const int64_t tiles = (N + rows_per_wg - 1) / rows_per_wg;
    const int per_cu = resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds);
    const int64_t cap = (int64_t)device_cu_count() * per_cu;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, cap));
    const int xvec = (aligned(x, XIn<XT>::kVecAlign) && ldx % 4 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, W, N, nb, x, ldx, y, ldy, xvec, PairRoute{});
    return check_launch("qmv");
}

// Lanes per row: whole waves for long rows, smaller segments for short rows
// so that lanes are not left idle (e.g. 24 blocks -> 8 lanes x 3).
template <class F, int B, int XU, int NW, class XT = float, int RPL = 1>
int32_t launch_lpr(const uint8_t* W, int64_t N, int nb, const XT* x, int64_t ldx, float* y, int64_t ldy,
                   hipStream_t st) {
    if (nb >= 64) return launch_b<F, B, 64, XU, NW, XT, RPL>(W, N, nb, x, ldx, y, ldy, st);
    if (nb >= 32) return launch_b<F, B, 32, XU, NW, XT, RPL>(W, N, nb, x, ldx, y, ldy, st);
    return launch_b<F, B, 8, XU, NW, XT, RPL>(W, N, nb, x, ldx, y, ldy, st);
}

template <class F, int XU, int NW, class XT = float, int RR = 1>
int32_t launch_c(const RowSegs& segs, int nb, const XT* x, hipStream_t st) {
    auto kern = qmv_kernel_c<F, XU, NW, 2, XT, RR>;
    const size_t lds =
        (size_t)nb * kXPad * sizeof(float) + (size_t)NW * RR * Contig<F>::kStepBytes;
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv", &dyn_max)) return e;
    if (lds > dyn_max) return fail(QMV_EINVAL, "qmv: %zu bytes of staged activations exceed the LDS", lds);
    const int64_t tiles = ((segs.end[segs.n - 1] + RR - 1) / RR + NW - 1) / NW;
    const int per_cu = resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds);
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, (int64_t)device_cu_count() * per_cu));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, segs, nb, x);
    return check_launch("qmv");
}

// XU 16-byte activation loads per thread stage K4 = K / 4 chunks with a
// workgroup of NW waves; past 8 per thread the staging loops instead.
template <class F, int NW, class XT = float, int RR = 1>
int32_t launch_c_xu(const RowSegs& segs, int nb, const XT* x, hipStream_t st) {
    const int per = (nb * 8 + 64 * NW - 1) / (64 * NW);
    if (per <= 1) return launch_c<F, 1, NW, XT, RR>(segs, nb, x, st);
    if (per <= 2) return launch_c<F, 2, NW, XT, RR>(segs, nb, x, st);
    if (per <= 4) return launch_c<F, 4, NW, XT, RR>(segs, nb, x, st);
    if (per <= 8) return launch_c<F, 8, NW, XT, RR>(segs, nb, x, st);
    return launch_c<F, 0, NW, XT, RR>(segs, nb, x, st);
}

// Batch 1 with whole 64-block steps and 16-byte aligned W and x: the
// contiguous-chunk kernel where it streams faster than per-block loads
// (measured on the 8B decode shapes, cache-cold):
//   Q8_0: matrices of >= 4096 rows or >= 256 blocks per row;
//   Q4_0/Q4_1 (closer to the VALU bound, where the LDS copy costs more):
//   2049..4096 rows, > 32768 rows, or >= 256 blocks per row.
// 16 waves per workgroup for long rows (one activation copy per CU) and
// for Q4 matrices of <= 4096 rows, else 8; fewer if the LDS does not fit.
template <class F, class XT = float>
bool try_launch_c(const RowSegs& segs, int nb, const XT* x, hipStream_t st, bool force, int32_t* rc) {
    if (nb % 64 || !aligned(x, XIn<XT>::kVecAlign) || segs.n < 1 || segs.n > kMaxSegs) return false;
    // 32-bit row indices and per-row buffer descriptors
    if (segs.end[segs.n - 1] >= ((int64_t)1 << 31) || (int64_t)nb * F::kBytes >= ((int64_t)1 << 31)) return false;
    for (int i = 0; i < segs.n; ++i)
        if (!aligned(segs.W[i], 16)) return false;
    const int64_t N = segs.end[segs.n - 1];
    const bool q8 = !F::kNibbles;
    const bool long_rows = nb >= 256;
    // Measured on the 8B steps (graph replays, same box): this kernel for
    // Q8_0 matrices of >= 4096 rows or long rows, and for Q4_x on long rows
    // (down), on 2049..4096 rows (q, o) and on > 32768 rows (lm_head); the
    // per-block kernel with two rows per lane is faster on the Q4_x k, v and
    // gate / up shapes.  Q4_x row sets of > 8192 rows take two rows per wave
    // step (4 waves).
    if (!force && (q8 ? !(N >= 4096 || long_rows) : !(long_rows || (N > 2048 && N <= 4096) || N > 32768)))
        return false;
    const size_t lds_x = (size_t)nb * kXPad * sizeof(float);
    if (!q8 && !long_rows && N > 8192 && lds_x + 4 * 2 * (size_t)Contig<F>::kStepBytes <= (size_t)kLdsMax) {
        *rc = launch_c_xu<F, 4, XT, 2>(segs, nb, x, st);
        return true;
    }
    int nw = (long_rows || (!q8 && N <= 4096)) ? 16 : 8;
    while (nw >= 4 && lds_x + (size_t)nw * Contig<F>::kStepBytes > (size_t)kLdsMax) nw /= 2;
    switch (nw) {
    case 16: *rc = launch_c_xu<F, 16, XT>(segs, nb, x, st); return true;
    case 8: *rc = launch_c_xu<F, 8, XT>(segs, nb, x, st); return true;
    case 4: *rc = launch_c_xu<F, 4, XT>(segs, nb, x, st); return true;
    default: return false;
    }
}

// Batch 1.  Workgroups of 8 waves when the staged activations (> 40 KB)
// allow few workgroups per CU, else 4 (more, smaller workgroups spread
// small matrices over every CU).  Activations are staged with straight-line
// 16-byte loads when 16-byte aligned: XU loads per thread cover
// K <= 16 * 64 * NW * XU / 4.
template <class F, class XT = float>
int32_t launch_b1(const uint8_t* W, int64_t N, int nb, const XT* x, int64_t ldx, float* y, int64_t ldy,
                  hipStream_t st) {
    int32_t rc;
    RowSegs one = {};
    one.W[0] = W;
    one.y[0] = y;
    one.end[0] = N;
    one.n = 1;
    if (try_launch_c<F, XT>(one, nb, x, st, false, &rc)) return rc;
    const size_t lds = (size_t)nb * kXPad * sizeof(float);
    const bool vec = aligned(x, XIn<XT>::kVecAlign);
    const int K4 = nb * 8;
    // Q4_x: two rows per lane (measured faster on every 8B shape it takes)
    constexpr int RPL = F::kNibbles ? 2 : 1;
    // 8 waves where x is large, and for Q8_0 (4096 x 4096: 6.0 -> 5.6 us);
    // Q4_x keeps 4 (q+k+v and lm_head were slower with 8)
    if (lds > 40 * 1024 || !F::kNibbles) {
        if (vec && K4 <= 2 * 512) return launch_lpr<F, 1, 2, 8, XT, RPL>(W, N, nb, x, ldx, y, ldy, st);
        if (vec && K4 <= 8 * 512) return launch_lpr<F, 1, 8, 8, XT, RPL>(W, N, nb, x, ldx, y, ldy, st);
        return launch_lpr<F, 1, 0, 8, XT, RPL>(W, N, nb, x, ldx, y, ldy, st);
    }
    if (vec && K4 <= 4 * 256) return launch_lpr<F, 1, 4, 4, XT, RPL>(W, N, nb, x, ldx, y, ldy, st);
    if (vec && K4 <= 16 * 256) return launch_lpr<F, 1, 16, 4, XT, RPL>(W, N, nb, x, ldx, y, ldy, st);
    return launch_lpr<F, 1, 0, 4, XT, RPL>(W, N, nb, x, ldx, y, ldy, st);
}

template <class F, class XT = float>
int32_t launch_batch(const uint8_t* W, int64_t N, int nb, const XT* x, int64_t ldx, int B, float* y,
                     int64_t ldy, hipStream_t st) {
    switch (B) {
    case 1: return launch_b1<F, XT>(W, N, nb, x, ldx, y, ldy, st);
    case 2: return launch_lpr<F, 2, 0, 8, XT>(W, N, nb, x, ldx, y, ldy, st);
    case 3: return launch_lpr<F, 3, 0, 8, XT>(W, N, nb, x, ldx, y, ldy, st);
    case 4: return launch_lpr<F, 4, 0, 8, XT>(W, N, nb, x, ldx, y, ldy, st);
    // 5..8 columns: the staged activations fill most of the LDS, so one
    // workgroup per CU; 16 waves share them (measured +13..26% at 8).
    case 5: return launch_lpr<F, 5, 0, 16, XT>(W, N, nb, x, ldx, y, ldy, st);
    case 6: return launch_lpr<F, 6, 0, 16, XT>(W, N, nb, x, ldx, y, ldy, st);
    case 7: return launch_lpr<F, 7, 0, 16, XT>(W, N, nb, x, ldx, y, ldy, st);
    default: return launch_lpr<F, 8, 0, 16, XT>(W, N, nb, x, ldx, y, ldy, st);
    }
}

int32_t check_common(const char* name, const void* W, int64_t N, int64_t K, const void* x, int64_t ldx,
                     int32_t batch, const void* y, int64_t ldy, int x_align = 4) {
    if (!W || !x || !y) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (N < 1) return fail(QMV_EINVAL, "%s: n_rows must be >= 1 (got %lld)", name, (long long)N);
    if (K < 32 || K % 32) return fail(QMV_EINVAL, "%s: n_cols must be a positive multiple of 32 (got %lld)", name, (long long)K);
    if (batch < 1 || batch > 8) return fail(QMV_EINVAL, "%s: batch must be in 1..8 (got %d)", name, batch);
    if (ldx < K) return fail(QMV_EINVAL, "%s: ldx (%lld) < n_cols (%lld)", name, (long long)ldx, (long long)K);
    if (ldy < N) return fail(QMV_EINVAL, "%s: ldy (%lld) < n_rows (%lld)", name, (long long)ldy, (long long)N);
    if (K / 32 > (1 << 26) || N > ((int64_t)1 << 40) / (K / 32))
        return fail(QMV_EINVAL, "%s: matrix too large (%lld x %lld)", name, (long long)N, (long long)K);
    if (!aligned(W, 4) || !aligned(y, 4))
        return fail(QMV_EALIGN, "%s: W and y must be 4-byte aligned", name);
    if (!aligned(x, x_align))
        return fail(QMV_EALIGN, "%s: x must be %d-byte aligned (its element size)", name, x_align);
    return QMV_OK;
}

template <class F>
constexpr qmv_fmt fmt_of() {
    return F::kBytes == 34 ? QMV_Q8_0 : (F::kBytes == 18 ? QMV_Q4_0 : QMV_Q4_1);
}

template <class XT> constexpr int32_t xtype_of();
template <> constexpr int32_t xtype_of<float>() { return QMV_X_F32; }
template <> constexpr int32_t xtype_of<_Float16>() { return QMV_X_F16; }
template <> constexpr int32_t xtype_of<__bf16>() { return QMV_X_BF16; }

// path: QMV_PATH_AUTO, QMV_PATH_FMA (the FMA kernels) or QMV_PATH_MFMA (the
// matrix-core kernel; QMV_EUNSUPPORTED where it does not apply).  XT: the
// activation element type (fp32, fp16 or bf16).
template <class F, class XT = float>
int32_t matvec(const char* name, const void* W, int64_t N, int64_t K, const XT* x, int64_t ldx, int32_t batch,
               float* y, int64_t ldy, void* stream, int32_t path = QMV_PATH_AUTO) {
    int32_t rc = check_common(name, W, N, K, x, ldx, batch, y, ldy, (int)sizeof(XT));
    if (rc != QMV_OK) return rc;
    const int nb = (int)(K / 32);
    // one activation row staged whole by the FMA kernels must fit in LDS;
    // beyond that the automatic choice takes the matrix cores where they apply
    const bool fma_fits = (int64_t)nb * kXPad * (int64_t)sizeof(float) <= kLdsMax;
    if (path == QMV_PATH_MFMA ||
        (path == QMV_PATH_AUTO && (use_mfma(fmt_of<F>(), N, nb, batch) || (!fma_fits && batch >= 2)))) {
        if (batch_matvec_mma(fmt_of<F>(), static_cast<const uint8_t*>(W), N, nb, x, xtype_of<XT>(), ldx, batch, y,
                             ldy, as_stream(stream), 0, &rc))
            return rc == QMV_OK ? ok() : rc;
        if (path == QMV_PATH_MFMA)
            return fail(QMV_EUNSUPPORTED,
                        "%s: the matrix-core path needs batch 2..8, n_cols a multiple of 256, W 16-byte aligned, "
                        "x aligned to 4 elements (16 bytes for fp32) and ldx a multiple of 4", name);
    }
    // The staged activation block (widened to fp32) must fit in LDS; wider
    // batches than fit are processed in column groups (each group re-reads
    // W).  16-bit activations take the same multi-column kernels: W is
    // streamed once per column group, not once per column.
    const int per_col = nb * kXPad * (int)sizeof(float);
    const int per_pass = std::max(1, std::min<int>(batch, kLdsMax / per_col));
    if (per_col > kLdsMax)
        return fail(QMV_EINVAL, "%s: n_cols %lld too large for one activation row in LDS", name, (long long)K);
    for (int b0 = 0; b0 < batch; b0 += per_pass) {
        const int bw = std::min(per_pass, batch - b0);
        rc = launch_batch<F, XT>(static_cast<const uint8_t*>(W), N, nb, x + b0 * ldx, ldx, bw, y + b0 * ldy, ldy,
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

// The grid is (range, group): group u serves the u-th distinct routed id
// (at most P = batch * top_k groups; the extra ones exit at once), and the
// ranges split each expert's row tiles so that ranges x expected groups
// fill the GPU once.  Expected groups: all P (spread), or the distinct ids
// that P uniformly routed pairs reach on average, E (1 - (1 - 1/E)^P).
template <class F, int BC, int LPR, int XU, int PD, bool SW, class XT>
int32_t launch_moe(const uint8_t* Wx, int64_t estride, int n_experts, int64_t N, int nb, const int32_t* ids,
                   int P, int top_k, const XT* x, int64_t xs_tok, int64_t xs_slot, float* y, int xvec,
                   bool spread, hipStream_t st) {
    constexpr int NW = 4;
    auto kern = moe_kernel<F, BC, LPR, NW, XU, PD, SW, XT>;
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv_moe", &dyn_max)) return e;
    const size_t lds = (size_t)BC * nb * kXPad * sizeof(float);
    if (lds > dyn_max)
        return fail(QMV_EINVAL, "qmv_moe: n_cols %d too large for one activation row in LDS", nb * 32);
    const int per_cu = resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds);
    const int64_t ntiles = (N + 64 / LPR - 1) / (64 / LPR);
    const double e = n_experts;
    const int64_t groups = std::max<int64_t>(
        1, std::min<int64_t>(std::min(P, n_experts),
                             spread ? P : (int64_t)std::ceil(e * (1.0 - std::pow(1.0 - 1.0 / e, (double)P)))));
    const int64_t gx = std::max<int64_t>(1, std::min<int64_t>(ntiles, (int64_t)device_cu_count() * per_cu / groups));
    hipLaunchKernelGGL(kern, dim3((unsigned)gx, (unsigned)P), dim3(64 * NW), lds, st, Wx, estride, n_experts, N, nb,
                       ids, P, top_k, x, xs_tok, xs_slot, y, xvec);
    return check_launch("qmv_moe");
}

// The grouping kernel runs where the per-pair route cannot stage its
// activations (rows of more than 16384 columns, or activations that are not
// 16-byte aligned).  Member columns per pass: one token routes to an expert
// once, so batch 1 needs one column.  At batches 2..8 a routed expert of 128 has 1.0 to 1.3
// members on average.  Measured on the 30B-A3B expert shapes (cache-cold):
// one column per pass, three steps in flight and a grid sized for the
// expected distinct experts win where the rows are long (2048 columns) or
// the batch is 8 (about 70 VGPRs: 7 waves per SIMD; an expert with two members
// streams twice, mostly from L2); on short rows at batch 2..4 there is
// too little work per workgroup for that, and two columns per pass over a
// grid sized for every pair measured faster.  Activations staged
// straight-line (XU 16-byte loads per thread) up to K = 8192.
template <class F, int LPR, int XU, bool SW, class XT>
int32_t launch_moe_bc(const uint8_t* Wx, int64_t estride, int n_experts, int64_t N, int nb, const int32_t* ids,
                      int batch, int top_k, const XT* x, int64_t xs_tok, int64_t xs_slot, float* y, int xvec,
                      hipStream_t st) {
    const int P = batch * top_k;
    const size_t per_col = (size_t)nb * kXPad * sizeof(float);
    if (batch > 1 && batch < 8 && nb < 64 && 2 * per_col + kMoeStaticLds <= (size_t)kLdsMax)
        return launch_moe<F, 2, LPR, XU, 2, SW, XT>(Wx, estride, n_experts, N, nb, ids, P, top_k, x, xs_tok, xs_slot,
                                                    y, xvec, true, st);
    return launch_moe<F, 1, LPR, XU, 3, SW, XT>(Wx, estride, n_experts, N, nb, ids, P, top_k, x, xs_tok, xs_slot, y,
                                                xvec, batch == 1, st);
}

// Every batch 1..8: pair p = token * top_k + slot is grid row p of the
// dense kernel on expert ids[p], with no prologue and no grouping.  An
// expert routed from several tokens (or twice by one) is streamed once per
// pair; the later streams find it mostly in L2 or the MALL, and the grid is
// the dense kernel's full persistent grid instead of a few steps per
// workgroup after a grouping prologue.
template <class F, int LPR, int XU, class XT, bool SW>
int32_t launch_moe_pairs(const uint8_t* Wx, int64_t estride, int n_experts, int64_t N, int nb, const int32_t* ids,
                         int batch, int top_k, const XT* x, int64_t xs_tok, int64_t xs_slot, float* y,
                         hipStream_t st) {
    constexpr int NW = 4;
    // Q4_x: two rows per lane, as the dense batch-1 kernel; SwiGLU: the
    // gate and up rows of an output row
    constexpr int RPL = (SW || F::kNibbles) ? 2 : 1;
    constexpr int OUT_RPL = SW ? 1 : RPL;      // output rows per lane
    auto kern = qmv_kernel<F, 1, LPR, RPL, XU, NW, 2, true, XT, SW>;
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv_moe", &dyn_max)) return e;
    const size_t lds = (size_t)nb * kXPad * sizeof(float);
    if (lds > dyn_max) return fail(QMV_EINVAL, "qmv_moe: %zu bytes of staged activations exceed the LDS", lds);
    const int per_cu = resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds);
    const int64_t tiles = (N + NW * (64 / LPR) * OUT_RPL - 1) / (NW * (64 / LPR) * OUT_RPL);
    const int pairs = batch * top_k;
    const int64_t gx = std::max<int64_t>(1, std::min<int64_t>(tiles, (int64_t)device_cu_count() * per_cu / pairs));
    const PairRoute route{ids, estride, xs_tok, xs_slot, top_k, n_experts};
    hipLaunchKernelGGL(kern, dim3((unsigned)gx, (unsigned)pairs), dim3(64 * NW), lds, st, Wx, N, nb, x,
                       (int64_t)nb * 32, y, N, 1, route);
    return check_launch("qmv_moe");
}

template <class F, int LPR, bool SW, class XT>
int32_t launch_moe_xu(const uint8_t* Wx, int64_t estride, int n_experts, int64_t N, int nb, const int32_t* ids,
                      int batch, int top_k, const XT* x, int64_t xs_tok, int64_t xs_slot, float* y, int xvec,
                      hipStream_t st) {
    const int K4 = nb * 8;   // 4-element chunks of one activation row; 256 threads
    // the per-pair route wherever the activations stage straight-line;
    // the grouping kernel otherwise
    const bool pairs = xvec != 0;
    if (pairs && K4 <= 4 * 256)
        return launch_moe_pairs<F, LPR, 4, XT, SW>(Wx, estride, n_experts, N, nb, ids, batch, top_k, x, xs_tok,
                                                   xs_slot, y, st);
    if (pairs && K4 <= 16 * 256)
        return launch_moe_pairs<F, LPR, 16, XT, SW>(Wx, estride, n_experts, N, nb, ids, batch, top_k, x, xs_tok,
                                                    xs_slot, y, st);
    if (K4 <= 2 * 256)
        return launch_moe_bc<F, LPR, 2, SW, XT>(Wx, estride, n_experts, N, nb, ids, batch, top_k, x, xs_tok, xs_slot, y,
                                                xvec, st);
    if (K4 <= 8 * 256)
        return launch_moe_bc<F, LPR, 8, SW, XT>(Wx, estride, n_experts, N, nb, ids, batch, top_k, x, xs_tok, xs_slot, y,
                                                xvec, st);
    return launch_moe_bc<F, LPR, 0, SW, XT>(Wx, estride, n_experts, N, nb, ids, batch, top_k, x, xs_tok, xs_slot, y,
                                            xvec, st);
}

// The combine kernel's grid: (row ranges, tokens).  Ranges x tokens fill
// the GPU once; a range holds at most kCombineRows rows (the row sums of
// all slots sit in LDS beside SC staged slot vectors).
constexpr int kCombineRows = 1024;

template <class F, int LPR, int NW>
int32_t launch_combine(const uint8_t* Wx, int64_t estride, int n_experts, int64_t N, int nb, const int32_t* ids,
                       const float* wts, int batch, int top_k, const float* x, int64_t xs_tok, int64_t xs_slot,
                       float* out, int xvec, hipStream_t st) {
    constexpr int PD = 3;
    constexpr int G = 64 / LPR;
    auto kern = moe_combine_kernel<F, LPR, NW, PD>;
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv_moe_combine", &dyn_max)) return e;
    const size_t per_col = (size_t)nb * kXPad * sizeof(float);
    const size_t sums_max = (size_t)top_k * (kCombineRows + 64) * sizeof(float);   // ranges round up to whole tiles
    if (per_col + sums_max > dyn_max)
        return fail(QMV_EINVAL, "qmv_moe_combine: n_cols %d too large for one activation row in LDS", nb * 32);
    const int SC = (int)std::min<size_t>((size_t)top_k, (dyn_max - sums_max) / per_col);
    const int64_t ntiles = (N + G - 1) / G;
    // residency for ranges of a few tiles (the row sums then take little LDS)
    const int per_cu = resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW,
                                    SC * per_col + (size_t)top_k * NW * G * sizeof(float));
    const int64_t min_ranges = (ntiles * G + kCombineRows - 1) / kCombineRows;
    const int64_t gx = std::max<int64_t>(
        min_ranges, std::min<int64_t>(ntiles, std::max<int64_t>(1, (int64_t)device_cu_count() * per_cu / batch)));
    const int64_t per_wg = (ntiles + gx - 1) / gx;
    const int rows_wg = (int)(per_wg * G);
    const size_t lds = SC * per_col + (size_t)top_k * rows_wg * sizeof(float);
    hipLaunchKernelGGL(kern, dim3((unsigned)gx, (unsigned)batch), dim3(64 * NW), lds, st, Wx, estride, n_experts, N, nb,
                       ids, wts, top_k, x, xs_tok, xs_slot, out, xvec, SC, rows_wg);
    return check_launch("qmv_moe_combine");
}

// Argument checks shared by the MoE entry points.  rows: rows of one
// expert matrix; n_out: rows of one output vector.
template <class F>
int32_t moe_check(const char* name, const void* Wx, int64_t estride, int32_t n_experts, int64_t rows, int64_t K,
                  const int32_t* ids, int32_t batch, int32_t top_k, const void* x, size_t x_elem, int64_t xs_tok,
                  int64_t xs_slot, const float* y) {
    if (!Wx || !ids || !x || !y) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (n_experts < 1) return fail(QMV_EINVAL, "%s: n_experts must be >= 1", name);
    if (rows < 1 || K < 32 || K % 32)
        return fail(QMV_EINVAL, "%s: bad matrix shape %lld x %lld", name, (long long)rows, (long long)K);
    if (batch < 1 || batch > 8) return fail(QMV_EINVAL, "%s: batch must be in 1..8 (got %d)", name, batch);
    if (top_k < 1 || top_k > 16) return fail(QMV_EINVAL, "%s: top_k must be in 1..16 (got %d)", name, top_k);
    const int64_t nb = K / 32;
    if (nb > (1 << 26) || rows > ((int64_t)1 << 40) / nb) return fail(QMV_EINVAL, "%s: matrix too large", name);
    const int64_t mbytes = rows * nb * F::kBytes;
    if (estride < mbytes || estride % 4)
        return fail(QMV_EINVAL, "%s: expert_stride_bytes (%lld) must be >= %lld and a multiple of 4", name,
                    (long long)estride, (long long)mbytes);
    if (n_experts > 1 && estride > ((int64_t)1 << 46) / (n_experts - 1)) return fail(QMV_EINVAL, "%s: experts too large", name);
    if (batch > 1 && xs_tok < K) return fail(QMV_EINVAL, "%s: x_stride_token must be >= n_cols", name);
    if (xs_tok < 0) return fail(QMV_EINVAL, "%s: x_stride_token must be >= 0", name);
    if (top_k > 1 && xs_slot != 0 && xs_slot < K) return fail(QMV_EINVAL, "%s: x_stride_slot must be 0 or >= n_cols", name);
    if (xs_slot < 0) return fail(QMV_EINVAL, "%s: x_stride_slot must be >= 0", name);
    if (!aligned(Wx, 4) || !aligned(y, 4) || !aligned(ids, 4))
        return fail(QMV_EALIGN, "%s: W_experts, the output and expert_ids must be 4-byte aligned", name);
    if (!aligned(x, x_elem)) return fail(QMV_EALIGN, "%s: x must be aligned to its %zu-byte elements", name, x_elem);
    const int64_t per_col = nb * kXPad * (int64_t)sizeof(float);
    if (per_col + kMoeStaticLds > kLdsMax)
        return fail(QMV_EINVAL, "%s: n_cols %lld too large for one activation row in LDS", name, (long long)K);
    return QMV_OK;
}

template <class XT>
int moe_xvec(const XT* x, int64_t xs_tok, int64_t xs_slot) {
    return (aligned(x, XIn<XT>::kVecAlign) && xs_tok % 4 == 0 && xs_slot % 4 == 0) ? 1 : 0;
}

// SW = false: y[p][i] = DEQ(W_e)[i] x_p (N rows per expert).  SW = true:
// every expert holds 2N rows and y[p][i] = SiLU(gate_i x_p) * (up_i x_p).
template <class F, bool SW, class XT = float>
int32_t moe(const char* name, const void* Wx, int64_t estride, int32_t n_experts, int64_t N, int64_t K,
            const int32_t* ids, int32_t batch, int32_t top_k, const XT* x, int64_t xs_tok, int64_t xs_slot, float* y,
            void* stream) {
    if (SW && N > ((int64_t)1 << 39)) return fail(QMV_EINVAL, "%s: n_ff too large", name);
    const int32_t rc = moe_check<F>(name, Wx, estride, n_experts, SW ? 2 * N : N, K, ids, batch, top_k, x, sizeof(XT),
                                    xs_tok, xs_slot, y);
    if (rc != QMV_OK) return rc;
    const int64_t nb = K / 32;
    const uint8_t* W8 = static_cast<const uint8_t*>(Wx);
    hipStream_t st = as_stream(stream);
    const int xvec = moe_xvec(x, xs_tok, xs_slot);
    if (nb >= 64)
        return launch_moe_xu<F, 64, SW, XT>(W8, estride, n_experts, N, (int)nb, ids, batch, top_k, x, xs_tok, xs_slot, y,
                                            xvec, st);
    if (nb >= 32)
        return launch_moe_xu<F, 32, SW, XT>(W8, estride, n_experts, N, (int)nb, ids, batch, top_k, x, xs_tok, xs_slot, y,
                                            xvec, st);
    return launch_moe_xu<F, 8, SW, XT>(W8, estride, n_experts, N, (int)nb, ids, batch, top_k, x, xs_tok, xs_slot, y,
                                       xvec, st);
}

template <class F>
int32_t moe_combine(const void* Wx, int64_t estride, int32_t n_experts, int64_t N, int64_t K, const int32_t* ids,
                    const float* wts, int32_t batch, int32_t top_k, const float* x, int64_t xs_tok, int64_t xs_slot,
                    float* out, void* stream) {
    const char* name = "qmv_moe_combine";
    if (!wts) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (!aligned(wts, 4)) return fail(QMV_EALIGN, "%s: weights must be 4-byte aligned", name);
    const int32_t rc = moe_check<F>(name, Wx, estride, n_experts, N, K, ids, batch, top_k, x, sizeof(float), xs_tok,
                                    xs_slot, out);
    if (rc != QMV_OK) return rc;
    const int64_t nb = K / 32;
    const uint8_t* W8 = static_cast<const uint8_t*>(Wx);
    hipStream_t st = as_stream(stream);
    const int xvec = moe_xvec(x, xs_tok, xs_slot);
    // at batch 1..2 the grid holds one row tile per workgroup: 8 waves give
    // each wave one (slot, tile) unit of a token's 8 slots
    const bool wide = batch <= 2;
    auto go = [&](auto lpr) {
        constexpr int L = decltype(lpr)::value;
        return wide ? launch_combine<F, L, 8>(W8, estride, n_experts, N, (int)nb, ids, wts, batch, top_k, x, xs_tok,
                                              xs_slot, out, xvec, st)
                    : launch_combine<F, L, 4>(W8, estride, n_experts, N, (int)nb, ids, wts, batch, top_k, x, xs_tok,
                                              xs_slot, out, xvec, st);
    };
    if (nb >= 64) return go(std::integral_constant<int, 64>{});
    if (nb >= 32) return go(std::integral_constant<int, 32>{});
    return go(std::integral_constant<int, 8>{});
}

// The entry points of one format, with the activation type chosen at run
// time: what a FormatOps table points to.
template <class F>
int32_t fmt_matvec(const char* name, const void* W, int64_t N, int64_t K, const void* x, int32_t x_type,
                   int64_t ldx, int32_t batch, float* y, int64_t ldy, void* stream, int32_t path) {
    switch (x_type) {
    case QMV_X_F32: return matvec<F, float>(name, W, N, K, static_cast<const float*>(x), ldx, batch, y, ldy, stream, path);
    case QMV_X_F16:
        return matvec<F, _Float16>(name, W, N, K, static_cast<const _Float16*>(x), ldx, batch, y, ldy, stream, path);
    case QMV_X_BF16:
        return matvec<F, __bf16>(name, W, N, K, static_cast<const __bf16*>(x), ldx, batch, y, ldy, stream, path);
    default: return fail(QMV_EINVAL, "%s: unknown activation type %d", name, (int)x_type);
    }
}

template <class F>
int32_t fmt_moe(const char* name, bool swiglu, const void* Wx, int64_t estride, int32_t E, int64_t N, int64_t K,
                const int32_t* ids, int32_t batch, int32_t top_k, const void* x, int32_t x_type, int64_t xs_tok,
                int64_t xs_slot, float* y, void* stream) {
    auto run = [&](auto xt) -> int32_t {
        using XT = decltype(xt);
        const XT* xp = static_cast<const XT*>(x);
        return swiglu ? moe<F, true, XT>(name, Wx, estride, E, N, K, ids, batch, top_k, xp, xs_tok, xs_slot, y, stream)
                      : moe<F, false, XT>(name, Wx, estride, E, N, K, ids, batch, top_k, xp, xs_tok, xs_slot, y, stream);
    };
    switch (x_type) {
    case QMV_X_F32: return run(float{});
    case QMV_X_F16: return run(_Float16{});
    case QMV_X_BF16: return run(__bf16{});
    default: return fail(QMV_EINVAL, "%s: unknown activation type %d", name, (int)x_type);
    }
}

template <class F>
bool fmt_group_contig(const RowSegs& segs, int nb, const float* x, hipStream_t st, bool force, int32_t* rc) {
    return try_launch_c<F, float>(segs, nb, x, st, force, rc);
}

template <class F>
const FormatOps& format_ops_for() {
    static const FormatOps ops = {fmt_matvec<F>, dequant<F>, fmt_moe<F>, moe_combine<F>, fmt_group_contig<F>};
    return ops;
}

}  // namespace
}  // namespace qmv
