// The batch-1 decode chain of qmv_chain as one persistent launch.
//
// A decode token is a sequence of matvecs, each streaming its weights once
// ("Economical Serving and the hanzo.ai Platform", Sec. 2.1: t = W/B), and
// each matvec's input is an earlier one's output.  Between two dependent
// matvecs every output of the first must be written and visible before the
// second reads its input.  This kernel runs a whole chain in one launch
// and keeps the weight stream going across those hand-overs where it can.
//
// Shape: one workgroup per compute unit, resident for the whole call, of
// 15 waves.
//  * 14 compute waves stream weights.  Their only global memory operations
//    are weight loads, issued straight into LDS (global_load_lds_dwordx4:
//    lane l writes 16 bytes at slot + 16 l) into a ring of P slots per wave.
//    A step is one row's 64-block window (2048 weights, 2176 / 1152 / 1280
//    bytes for Q8_0 / Q4_0 / Q4_1).  Each step's block for lane l is read
//    back from the slot, decoded, dotted with the lane's 32 activations
//    (held in registers, taken from the staged x when the window changes),
//    reduced across the wave, and its window partial goes to LDS.
//  * 1 control wave does everything that must wait: it sums each row's
//    window partials (in window order) and writes the outputs with
//    device-coherent stores, meets the other workgroups at a grid barrier
//    before a level that reads outputs of an earlier one, and stages that
//    level's x into LDS (device-coherent loads straight into LDS).  It never
//    has weight loads in flight, so none of its waits waits for them.
//
// Why the roles are split: a wave's memory operations complete in order
// (one counter), so a wave with weight loads in flight cannot wait for a
// barrier word or an activation load without also waiting for its weight
// loads.  Here only the control wave waits for such things.
//
// What a hand-over costs (measured on the MI355X, one workgroup per CU):
// a device-coherent load takes about 0.1 us when the memory system is
// quiet and 1.6 us while the GPU streams; a bare grid hand-over of 16
// outputs per workgroup (store, acknowledge, flag, poll, load) costs about
// 5 us, and 4.3 us even when each output carries its own generation tag
// and the consumer polls the data directly.  A kernel boundary between two
// dependent launches in a HIP graph costs about 2.9 us.  So the compute
// waves prefetch only kDecAhead steps of a later level before its x is
// staged (deeper prefetch loads the memory system and slows the
// hand-over), and the batch-1 decode step itself is faster as one launch
// per dependency level (qmv_chain's single-level groups, the dense
// entry points) than as one chain; this kernel is the faster way to run a
// dependent chain in a single call (2.01 ms against 2.32 ms for per-stage
// cursors with a two-level atomic barrier, 8B Q8_0 step).
//
// Grid barrier: a flag word per workgroup in the workspace.  A workgroup
// that has written level L's outputs (its stores acknowledged) stores its
// barrier count; a waiter reads all flags until each has reached the count.
// The counts continue across calls (each call reads its own flag first), so
// the words need no reset; every call uses the same grid (one workgroup per
// compute unit).  The wait is bounded (50 ms): on timeout the error word is
// set and the workgroup goes on, so a grid that is not co-resident ends
// instead of hanging.
//
// Arithmetic per row: lane l of window w computes block 64 w + l's term
// (the per-format factors and Term<F> of the other kernels), the wave sums
// the 64 terms in a fixed tree (segment_sum), and the row is the sum of
// its window partials in window order: deterministic, within the accuracy
// bound, and not bitwise the per-matvec kernels (they accumulate a lane's
// blocks across windows before the tree).
#include "qmv_block_decode.h"

namespace qmv {
namespace {

constexpr int kDecCompute = 14;                  // compute waves per workgroup
constexpr int kDecWaves = kDecCompute + 1;       // + the control wave (wave 0)
constexpr int kDecMaxLevels = 36;
constexpr int kWinCols = 2048;                   // columns per window (64 blocks)
constexpr int kFlagWord = 9216;                  // flags: workspace words [9216, 10240)
constexpr int kMaxFlags = 1024;
constexpr int kErrWord = 2;
constexpr int kPolNT = 2;                        // cache policy: non-temporal (weights)
constexpr int kPolSc1 = 16;                      // cache policy: device-coherent (activations)
constexpr unsigned long long kDecWaitTicks = 5000000ull;   // 50 ms of the 100 MHz real-time counter

struct DecLevel {              // one dependency level: up to 4 matrices reading one x
    const uint8_t* W[kMaxSegs];
    float* y[kMaxSegs];
    const float* x;
    int32_t end[kMaxSegs];     // cumulative rows: matrix k holds rows [end[k-1], end[k])
    int16_t nseg;
    int16_t nwin;              // n_cols / 2048
    int16_t wait;              // grid barrier before staging x
    int16_t pad;
};

struct DecArgs {
    DecLevel lv[kDecMaxLevels];
    unsigned* ws;              // workspace words
    int32_t n;                 // levels
    int32_t ahead;             // steps per wave issued into a later level before its x is staged
    int32_t xs_floats;         // LDS floats for the staged x
    int32_t part_floats;       // LDS floats for the window partials
};

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ unsigned load_agent(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The 32 floats at LDS address p (16-byte aligned) into v, read in one asm
// block that also waits for them: written as plain loads, the compiler
// makes every LDS read of the kernel wait for all loads into LDS in flight
// (it cannot tell the staged x from the weight ring), which would drain the
// ring at each window change.
__device__ __forceinline__ void lds_read32(const float* p, float (&v)[32]) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const float*)p);
    f4 q0, q1, q2, q3, q4, q5, q6, q7;
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:16\n\t"
        "ds_read_b128 %2, %8 offset:32\n\t"
        "ds_read_b128 %3, %8 offset:48\n\t"
        "ds_read_b128 %4, %8 offset:64\n\t"
        "ds_read_b128 %5, %8 offset:80\n\t"
        "ds_read_b128 %6, %8 offset:96\n\t"
        "ds_read_b128 %7, %8 offset:112\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3), "=&v"(q4), "=&v"(q5), "=&v"(q6), "=&v"(q7)
        : "v"(a)
        : "memory");
    const f4 q[8] = {q0, q1, q2, q3, q4, q5, q6, q7};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[4 * i] = q[i].x;
        v[4 * i + 1] = q[i].y;
        v[4 * i + 2] = q[i].z;
        v[4 * i + 3] = q[i].w;
    }
}

// Workgroup barrier without a memory fence: the LDS operations of this wave
// are complete (lgkmcnt 0), its global operations are not waited for (the
// compute waves' weight loads stay in flight).
__device__ __forceinline__ void wg_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <class F>
struct DecStep {
    static constexpr int kBytes = 64 * F::kBytes;              // 2176 / 1152 / 1280
    static constexpr int kChunks = kBytes / 16;                 // 136 / 72 / 80
    static constexpr int kLoads = (kChunks + 63) / 64;          // 3 / 2 / 2
    static_assert(kBytes % 16 == 0, "whole 16-byte chunks");
};

// Rows [r0, r1) of a level that workgroup b owns: contiguous, ceil(R / G) each.
__device__ __forceinline__ void wg_rows(const DecLevel& L, int G, int b, int& r0, int& r1) {
    const int R = L.end[L.nseg - 1];
    const int per = (R + G - 1) / G;
    r0 = min(R, b * per);
    r1 = min(R, r0 + per);
}

template <class F, int P>
__global__ __launch_bounds__(64 * kDecWaves) void decode_kernel(const DecArgs args) {
    using S = DecStep<F>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    float* xs = reinterpret_cast<float*>(lds);                              // staged x [xs_floats]
    float* part = xs + args.xs_floats;                                      // window partials
    uint8_t* ring = reinterpret_cast<uint8_t*>(part + args.part_floats);    // [14][P][S::kBytes]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int n = args.n;

    if (wave == 0) {
        // ------------------------------------------------------------ control
        unsigned* flags = args.ws + kFlagWord;
        unsigned* err = args.ws + kErrWord;
        const unsigned base = load_agent(flags + b);     // this call's starting count
        unsigned count = 0;
        bool broken = false;
        for (int L = 0; L < n; ++L) {
            const DecLevel& lv = args.lv[L];
            if (L > 0 && lv.wait) {
                // every workgroup's outputs of the earlier levels are written
                ++count;
                if (lane == 0) store_agent(flags + b, base + count);
                if (!broken) {
                    const unsigned target = base + count;
                    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
                    while (true) {
                        bool ok = true;
                        for (int j = lane; j < G; j += 64) ok = ok && (int)(load_agent(flags + j) - target) >= 0;
                        if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
                        if (__builtin_amdgcn_s_memrealtime() - t0 > kDecWaitTicks) {
                            if (lane == 0) store_agent(err, 1u);
                            broken = true;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
            }
            // stage x of this level: device-coherent 16-byte loads straight into LDS
            const int K = lv.nwin * kWinCols;
            const uint8_t* xg = reinterpret_cast<const uint8_t*>(lv.x);
            for (int c0 = 0; c0 < K / 4; c0 += 64)
                __builtin_amdgcn_global_load_lds(xg + 16 * (c0 + lane), (lds_ptr)(xs + 4 * c0), 16, 0, kPolSc1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            wg_barrier();   // B: x staged
            wg_barrier();   // A: the compute waves' partials of this level are in LDS
            int r0, r1;
            wg_rows(lv, G, b, r0, r1);
            const int nw = lv.nwin;
            for (int r = r0 + lane; r < r1; r += 64) {
                const float* p = part + (r - r0) * nw;
                float v = p[0];
                for (int w = 1; w < nw; ++w) v += p[w];
                int k = 0;
                while (k + 1 < lv.nseg && r >= lv.end[k]) ++k;
                store_agent(lv.y[k] + (r - (k ? lv.end[k - 1] : 0)), v);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // outputs acknowledged before the next flag
        }
        return;
    }

    // ---------------------------------------------------------------- compute
    const int c = wave - 1;
    uint8_t* my_ring = ring + c * P * S::kBytes;

    // Load cursor over this wave's steps: items c, c + 14, ... of each level
    // in turn, item i being row r0 + i / nwin, window i % nwin.  All
    // divisions and argument reads happen once per level; a step advances
    // (row, window, matrix) with a few adds.
    struct Cursor {
        int L;                    // level (n: past the end)
        int row, r1;              // row (level-wide index) and the workgroup's end row
        int w, nw, dq, dr;        // window; windows per row; 14 = dq * nw + dr
        int seg, seg_lo, seg_hi;  // the row's matrix and its rows [seg_lo, seg_hi)
        const uint8_t* segW;
        int64_t pitch;            // bytes per row
    } lc;
    auto set_seg = [&](Cursor& k) {
        const DecLevel& lv = args.lv[k.L];
        while (k.row >= k.seg_hi) {
            ++k.seg;
            k.seg_lo = k.seg_hi;
            k.seg_hi = lv.end[k.seg];
            k.segW = lv.W[k.seg];
        }
    };
    // positions k at its first item of level L or later (k.L = n past the end)
    auto enter = [&](Cursor& k, int L) {
        for (; L < n; ++L) {
            const DecLevel& lv = args.lv[L];
            int r0, r1;
            wg_rows(lv, G, b, r0, r1);
            const int nw = lv.nwin;
            if (c < (r1 - r0) * nw) {
                k.L = L;
                k.row = r0 + c / nw;
                k.r1 = r1;
                k.w = c % nw;
                k.nw = nw;
                k.dq = kDecCompute / nw;
                k.dr = kDecCompute % nw;
                k.seg = 0;
                k.seg_lo = 0;
                k.seg_hi = lv.end[0];
                k.segW = lv.W[0];
                k.pitch = (int64_t)nw * S::kBytes;
                set_seg(k);
                return;
            }
        }
        k.L = n;
    };
    auto advance = [&](Cursor& k) {
        k.w += k.dr;
        k.row += k.dq;
        if (k.w >= k.nw) {
            k.w -= k.nw;
            ++k.row;
        }
        if (k.row >= k.r1) enter(k, k.L + 1);
        else set_seg(k);
    };
    auto addr = [&](const Cursor& k) -> const uint8_t* {
        return k.segW + (int64_t)(k.row - k.seg_lo) * k.pitch + (int64_t)k.w * S::kBytes;
    };
    enter(lc, 0);
    // Ring accounting: steps issued and computed by this wave; step t uses
    // slot t % P.  A step of a later level than the one being computed is
    // issued only while fewer than `ahead_max` such steps are in flight:
    // with few weight loads in flight the memory system is quiet when the
    // control wave's hand-over runs (its dependent round trips take a
    // fraction of their loaded latency), and the first steps of the next
    // level are already on their way.
    int issued = 0, computed = 0, ahead = 0;
    const int ahead_max = args.ahead;
    auto try_issue = [&](int Lc) -> bool {
        if (issued - computed >= P || lc.L >= n) return false;
        if (lc.L > Lc) {
            if (ahead >= ahead_max) return false;
            ++ahead;
        }
        const uint8_t* a = addr(lc);
        advance(lc);
        uint8_t* dst = my_ring + (issued % P) * S::kBytes;
#pragma unroll
        for (int k = 0; k < S::kLoads; ++k) {
            if (64 * k + 64 <= S::kChunks || 64 * k + lane < S::kChunks)
                __builtin_amdgcn_global_load_lds(a + 16 * (64 * k + lane), (lds_ptr)(dst + 1024 * k), 16, 0, kPolNT);
        }
        ++issued;
        return true;
    };
    // Waits until the oldest step in flight has landed: every later step's
    // loads may still be outstanding (loads complete in order).
    auto wait_oldest = [&]() {
        const int later = issued - computed - 1;
        static_assert(P <= 6, "wait table");
        switch (later) {
        case 5: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * S::kLoads) : "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * S::kLoads) : "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * S::kLoads) : "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * S::kLoads) : "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(1 * S::kLoads) : "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        }
    };
    // before the first x is staged: the first level's steps (and no more
    // than ahead_max of a later level, in case this wave has none here)
    while (try_issue(0)) {
    }

    for (int L = 0; L < n; ++L) {
        wg_barrier();   // B: x of level L staged
        ahead = 0;      // steps of level L issued earlier are now this level's
        while (try_issue(L)) {
        }
        const DecLevel& lv = args.lv[L];
        int r0, r1;
        wg_rows(lv, G, b, r0, r1);
        const int nw = lv.nwin;
        const int items = (r1 - r0) * nw;
        const int dr = kDecCompute % nw;
        int w = c % nw;
        int cur_w = -1;
        float xv[32];
        for (int i = c; i < items; i += kDecCompute) {
            if (w != cur_w) {
                lds_read32(xs + w * kWinCols + 32 * lane, xv);
                cur_w = w;
            }
            wait_oldest();
            const uint8_t* slotp = my_ring + (computed % P) * S::kBytes;
            typename F::Raw raw;
            F::from_lds(slotp, lane, raw);
            float d, m;
            uint32_t cd[8];
            F::decode(raw, d, m, cd);
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float f[4];
                chunk_codes<F>(cd, q, d, m, f);
                s = __builtin_fmaf(f[0], xv[4 * q], s);
                s = __builtin_fmaf(f[1], xv[4 * q + 1], s);
                s = __builtin_fmaf(f[2], xv[4 * q + 2], s);
                s = __builtin_fmaf(f[3], xv[4 * q + 3], s);
            }
            const float tot = segment_sum<64>(Term<F>::add(0.f, d, m, s));
            if (lane == 0) part[i] = tot;   // row r0 + i / nw, window w
            // the slot's LDS reads are complete (their values are used
            // above); it can take the next step
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            ++computed;
            try_issue(L);
            w += dr;
            if (w >= nw) w -= nw;
        }
        wg_barrier();   // A: this wave's partials of level L are in LDS
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no LDS write may land after the workgroup ends
}

// Steps per compute wave issued into a later level before its x is staged.
// Measured on the 8B decode step (Q8_0, one call of 225 stages): 0 / 1 / 2 /
// 3 steps gave 2.12 / 2.01 / 2.01 / 2.06 ms.  A device-coherent load takes
// 0.1 us on a quiet memory system and 1.6 us while the GPU streams, and the
// hand-over is a chain of such round trips, so deeper prefetch slows it.
constexpr int kDecAhead = 1;

template <class F, int P>
int32_t launch_decode(DecArgs& a, hipStream_t st) {
    auto kern = decode_kernel<F, P>;
    const size_t lds = (size_t)(a.xs_floats + a.part_floats) * sizeof(float) +
                       (size_t)kDecCompute * P * DecStep<F>::kBytes;
    size_t dyn_max = 0;
    if (const int32_t e = lds_limit(reinterpret_cast<const void*>(kern), kLdsMax, "qmv_chain", &dyn_max)) return e;
    if (lds > dyn_max) return fail(QMV_EINVAL, "qmv_chain: %zu bytes of LDS needed", lds);
    const int G = device_cu_count();
    hipLaunchKernelGGL(kern, dim3(G), dim3(64 * kDecWaves), lds, st, a);
    return check_launch("qmv_chain");
}

template <class F>
bool decode_chain_f(const qmv_chain_stage* stages, int32_t n_stages, unsigned* ws, hipStream_t st, int32_t* rc) {
    const int G = device_cu_count();
    if (G > kMaxFlags) return false;
    // group the stages into levels: consecutive stages reading one x with
    // the same width, the later ones not waiting, at most kMaxSegs
    struct Lv {
        int first, count;
    };
    Lv lv[4096];
    int nl = 0;
    int max_cols = 0;
    for (int s = 0; s < n_stages;) {
        const qmv_chain_stage& q = stages[s];
        if (q.n_cols % kWinCols || !aligned(q.W, 16) || !aligned(q.x, 16) || nl >= 4096) return false;
        int k = 1;
        while (s + k < n_stages && k < kMaxSegs && !stages[s + k].wait && stages[s + k].x == q.x &&
               stages[s + k].n_cols == q.n_cols && aligned(stages[s + k].W, 16))
            ++k;
        lv[nl++] = {s, k};
        max_cols = std::max<int>(max_cols, (int)q.n_cols);
        s += k;
    }
    // LDS: staged x, window partials (largest rows-per-workgroup x windows), ring
    int64_t part = 0;
    for (int i = 0; i < nl; ++i) {
        int64_t rows = 0;
        for (int k = 0; k < lv[i].count; ++k) rows += stages[lv[i].first + k].n_rows;
        part = std::max<int64_t>(part, (rows + G - 1) / G * (stages[lv[i].first].n_cols / kWinCols));
    }
    part = (part + 3) / 4 * 4;
    constexpr int P = F::kNibbles ? 5 : 3;
    const size_t need = (size_t)(max_cols + part) * sizeof(float) + (size_t)kDecCompute * P * DecStep<F>::kBytes;
    if (need > (size_t)kLdsMax) return false;
    for (int l0 = 0; l0 < nl; l0 += kDecMaxLevels) {
        DecArgs a = {};
        a.n = std::min(kDecMaxLevels, nl - l0);
        a.ws = ws;
        a.xs_floats = max_cols;
        a.ahead = kDecAhead;
        a.part_floats = (int32_t)part;
        for (int i = 0; i < a.n; ++i) {
            const Lv& L = lv[l0 + i];
            DecLevel& d = a.lv[i];
            int64_t rows = 0;
            for (int k = 0; k < L.count; ++k) {
                const qmv_chain_stage& q = stages[L.first + k];
                d.W[k] = static_cast<const uint8_t*>(q.W);
                d.y[k] = q.y;
                rows += q.n_rows;
                d.end[k] = (int32_t)rows;
            }
            d.x = stages[L.first].x;
            d.nseg = (int16_t)L.count;
            d.nwin = (int16_t)(stages[L.first].n_cols / kWinCols);
            d.wait = (int16_t)((i > 0 && stages[L.first].wait) ? 1 : 0);   // a kernel boundary orders the first
        }
        *rc = launch_decode<F, P>(a, st);
        if (*rc != QMV_OK) return true;
    }
    return true;
}

}  // namespace

bool decode_chain(qmv_fmt fmt, const qmv_chain_stage* stages, int32_t n_stages, unsigned* ws, hipStream_t st,
                  int32_t* rc) {
    switch (fmt) {
    case QMV_Q8_0: return decode_chain_f<Q8_0>(stages, n_stages, ws, st, rc);
    case QMV_Q4_0: return decode_chain_f<Q4_0>(stages, n_stages, ws, st, rc);
    case QMV_Q4_1: return decode_chain_f<Q4_1>(stages, n_stages, ws, st, rc);
    default: return false;
    }
}

}  // namespace qmv
