// A chain of batch-1 block-quantized matvecs in one persistent launch.
//
// Decode runs one matvec after another ("Economical Serving and the hanzo.ai
// Platform", Sec. 2.1: a token is one stream of the resident weights); at
// batch 1 each matvec is a few microseconds of HBM traffic, comparable to
// the fixed cost of a kernel launch on this GPU (about 2.5 us back to back).
// qmv_chain runs a list of stages, y_s = DEQ(W_s) x_s, inside one launch:
// the grid stays resident, each wave streams its row tiles stage after
// stage, and the loads of a stage's first blocks are issued while the
// previous stage is still being computed.  A stage marked `wait` reads
// outputs of earlier stages: before it stages its activations every
// workgroup meets at a grid barrier (all earlier outputs written through to
// device-coherent memory).  The wave's wait before it arrives covers every
// outstanding memory operation, so the weight loads it issued for the
// stage's first step land before the barrier (they are in registers when
// it ends) rather than overlapping it: only their issue is early.  Stages
// without `wait` start as soon as each workgroup is done.
//
// The per-stage arithmetic is the batch-1 dense kernel's (64 lanes per row
// segment, fixed reduction order), so each stage's output equals a
// qmv_q8_0 / qmv_q4_0 / qmv_q4_1 call on a matrix of >= 64 blocks per row
// bitwise.
#include <mutex>
#include <type_traits>

#include "qmv_block_decode.h"

// The barrier words of qmv_chain_noalloc, held by the library: a file-scope
// device array, so every GPU the library runs on holds one copy (at its own
// address) until the process ends.  Host code never passes this name to a
// kernel or a copy (in host code it is only a stand-in for the symbol): it
// looks the device address up with hipGetSymbolAddress once per device and
// uses that pointer.
static __device__ __align__(256) unsigned scratch[QMV_CHAIN_WORKSPACE_BYTES / 4];

namespace qmv {
namespace {

constexpr int kChainMaxStages = 64;

struct ChainStage {        // 40 bytes in the kernel arguments
    const uint8_t* W;
    const float* x;
    float* y;
    int32_t N;
    int16_t nb;
    int8_t wait;
    int8_t xvec;           // x is 16-byte aligned
    int32_t off;           // wave (of the grid's waves) that takes row 0
};

struct ChainArgs {
    ChainStage st[kChainMaxStages];
    unsigned* bar;         // barrier words (top at [0], groups 4 KB apart), [2] error flag
    int32_t n;
    int32_t nwg;
    int32_t xfloats;       // LDS floats of staged activations; the weight copies follow
};

constexpr int kSc1 = 16;                     // buffer cache-policy operand: device-scope coherent
constexpr int kGroups = 8;                   // barrier groups: one per XCD under round-robin dispatch
constexpr int kGroupWords = 1024;            // 4 KB between the barrier words
constexpr unsigned long long kWaitTicks = 5000000ull;   // 50 ms of the 100 MHz real-time counter

// Cross-workgroup data of a chain (stage outputs, barrier words) moves only
// through device-scope coherent accesses: stores and loads with sc1, which
// write through and read past the per-XCD L2 caches.  No fence is needed,
// so no wave ever writes back or invalidates a whole L2 (an agent-scope
// fence does both, and at every stage that costs more than the matvecs).

__device__ __forceinline__ unsigned load_coherent(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_coherent(unsigned* p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid-wide barrier of the nwg resident workgroups, in two levels so that
// no single word takes more than nwg/8 + 1 arrivals (same-word atomics
// serialize in the memory system) or pollers.  Each barrier word holds
// generation << 16 | arrivals, so one fetch-add returns both the arrival
// order and the generation to wait out.  Workgroup b belongs to group
// b % 8; the last arrival of a group arrives at the top word; the last
// arrival at the top starts the next generation of the top and of every
// group word (adding 65536 - members resets the arrivals in the same
// atomic), and the others poll their group's word.  Words are left ready
// for the next barrier and the next call.  Every wave first waits for its
// own outstanding memory operations, its sc1 output stores among them.
// The wait is bounded: on timeout bar[2] is set and false is returned; the
// caller then skips its later barriers, so a broken launch ends quickly.
__device__ __forceinline__ bool grid_barrier_thread0(unsigned* bar, unsigned nwg) {
    const unsigned ng = nwg < kGroups ? nwg : kGroups;
    const unsigned g = blockIdx.x % kGroups;
    const unsigned members = nwg / kGroups + (g < nwg % kGroups ? 1u : 0u);
    unsigned* gw = bar + kGroupWords * (g + 1);
    const unsigned old = add_coherent(gw, 1u);
    const unsigned gen = old >> 16;
    if ((old & 0xFFFFu) == members - 1) {
        const unsigned t = add_coherent(bar, 1u);
        if ((t & 0xFFFFu) == ng - 1) {
            add_coherent(bar, 65536u - ng);
            for (unsigned k = 0; k < ng; ++k)
                add_coherent(bar + kGroupWords * (k + 1), 65536u - (nwg / kGroups + (k < nwg % kGroups ? 1u : 0u)));
            return true;
        }
    }
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while ((load_coherent(gw) >> 16) == gen) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
            __hip_atomic_store(&bar[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
    }
    return true;
}

// Stages one activation vector x[0..32 nb) into LDS as xs[block][36],
// reading it with device-coherent loads: x may have been written by other workgroups
// earlier in the same launch.  Same layout and batching as the dense
// kernel's staging; loads past the end of x read 0 and are not stored.
template <int NT>
__device__ __forceinline__ void stage_x_coherent(const float* x, int nb, float* xs, bool vec) {
    const int K = nb * 32;
    const int tid = threadIdx.x;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, K * 4, 0x00020000);
    if (vec) {
        const int K4 = K >> 2;
        auto put = [&](int c, int4 v) {
            const int e = 4 * c;
            *reinterpret_cast<int4*>(xs + (e >> 5) * kXPad + (e & 31)) = v;
        };
        auto get = [&](int c) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * c, 0, kSc1);
            return int4{v[0], v[1], v[2], v[3]};
        };
        for (int c0 = tid; c0 < K4; c0 += 4 * NT) {
            const int c1 = c0 + NT, c2 = c0 + 2 * NT, c3 = c0 + 3 * NT;
            const int4 v0 = get(c0), v1 = get(c1), v2 = get(c2), v3 = get(c3);
            put(c0, v0);
            if (c1 < K4) put(c1, v1);
            if (c2 < K4) put(c2, v2);
            if (c3 < K4) put(c3, v3);
        }
    } else {
        auto put = [&](int e, uint32_t v) { reinterpret_cast<uint32_t*>(xs)[(e >> 5) * kXPad + (e & 31)] = v; };
        auto get = [&](int e) { return __builtin_amdgcn_raw_buffer_load_b32(r, 4 * e, 0, kSc1); };
        for (int e0 = tid; e0 < K; e0 += 4 * NT) {
            const int e1 = e0 + NT, e2 = e0 + 2 * NT, e3 = e0 + 3 * NT;
            const uint32_t v0 = get(e0), v1 = get(e1), v2 = get(e2), v3 = get(e3);
            put(e0, v0);
            if (e1 < K) put(e1, v1);
            if (e2 < K) put(e2, v2);
            if (e3 < K) put(e3, v3);
        }
    }
    __syncthreads();
}

// CONTIG: every stage has whole 64-block steps and 16-byte aligned W, and
// its weights arrive as whole 16-byte chunks (non-temporal) copied through
// a per-wave LDS scratch, as in the contiguous dense kernel.  Otherwise
// each lane loads its own block.
template <class F, int NW, bool CONTIG>
__global__ __launch_bounds__(64 * NW) void chain_kernel(const ChainArgs args) {
    constexpr int LPR = 64;
    extern __shared__ __attribute__((aligned(16))) float lds[];   // 16-byte aligned after any static LDS
    float* xs = lds;
    const int li = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w0 = (int)blockIdx.x * NW + wave;        // rows < 2^30, waves < 2^16: int
    const int wstride = (int)gridDim.x * NW;
    const int n = args.n;
    using C = Contig<F>;
    using Raw = typename std::conditional<CONTIG, typename C::Chunks, typename F::Raw>::type;
    uint8_t* scratch = reinterpret_cast<uint8_t*>(lds + args.xfloats) + wave * C::kStepBytes;

    // The load cursor runs one step ahead of the compute cursor, across
    // stage boundaries.  A step is (stage, row, t): lane li handles block
    // li + 64 t of the row.  Row r of stage s goes to wave (off_s + r) mod
    // wstride: the stages' rows continue one round-robin, so short stages
    // do not all land on the first waves.
    auto first_row = [&](int s) -> int { return (w0 - args.st[s].off + wstride) % wstride; };
    int ls = 0;
    int lrow = first_row(0);
    int lt = 0;
    auto skip_empty = [&](int& s, int& row, int& t) {
        while (s < n && row >= args.st[s].N) {
            ++s;
            if (s < n) row = first_row(s);
            t = 0;
        }
    };
    auto advance = [&](int& s, int& row, int& t) {
        const int T = (args.st[s].nb + LPR - 1) / LPR;
        if (++t == T) { t = 0; row += wstride; }
        skip_empty(s, row, t);
    };
    auto load_next = [&](Raw& r) {
        // past the last step: re-read a block already loaded (in cache)
        const int s = ls < n ? ls : n - 1;
        const ChainStage& st = args.st[s];
        const int64_t row = ls < n ? lrow : min(w0, st.N - 1);
        const int t = ls < n ? lt : 0;
        if constexpr (CONTIG) {
            C::fetch(st.W + (row * st.nb + 64 * t) * F::kBytes, li, r);
        } else {
            const int j = min(li + LPR * t, (int)st.nb - 1);
            F::fetch(st.W, row * st.nb + j, r);
        }
        if (ls < n) advance(ls, lrow, lt);
    };
    auto stage_x = [&](int s) {
        const ChainStage& st = args.st[s];
        stage_x_coherent<64 * NW>(st.x, st.nb, xs, st.xvec != 0);
    };
    float acc = 0.f;
    auto compute = [&](int s, int row, int t, const Raw& r) {
        const ChainStage& st = args.st[s];
        const int nb = st.nb;
        const int j = li + LPR * t;
        const bool valid = j < nb;
        const int jc = valid ? j : nb - 1;
        float d, m;
        uint32_t c[8];
        if constexpr (CONTIG) {
            typename F::Raw blk;
            C::to_block(r, scratch, li, blk);
            F::decode(blk, d, m, c);
        } else {
            F::decode(r, d, m, c);
        }
        float q[32];
        codes_to_float<F>(c, d, m, q);
        float sdot[1] = {0.f};
        dot_cols<1>(q, xs + jc * kXPad, nb * kXPad, sdot, 1);
        const float upd = Term<F>::add(acc, d, m, sdot[0]);
        acc = valid ? upd : acc;
        if (t == (nb + LPR - 1) / LPR - 1) {
            const float tot = segment_sum<LPR>(acc);
            if (li == 0) __hip_atomic_store(st.y + row, tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            acc = 0.f;
        }
    };

    int cs = 0;
    int crow = first_row(0);
    int ct = 0;
    skip_empty(ls, lrow, lt);
    skip_empty(cs, crow, ct);
    Raw bufA, bufB;
    load_next(bufA);
    stage_x(0);

    // The wave's remaining steps of stage s.  run_from_A: the next step's
    // loads are in bufA (B: in bufB); each returns true when, on leaving the
    // stage, the next step's loads are in bufB.  The two buffers alternate
    // in straight-line code, so the compiler waits only for the one in use.
    auto run_from_A = [&](int s) -> bool {
        if (cs != s) return false;
        while (true) {
            load_next(bufB);
            __builtin_amdgcn_sched_barrier(0);   // issue the next loads before using bufA
            compute(cs, crow, ct, bufA);
            advance(cs, crow, ct);
            if (cs != s) return true;
            load_next(bufA);
            __builtin_amdgcn_sched_barrier(0);
            compute(cs, crow, ct, bufB);
            advance(cs, crow, ct);
            if (cs != s) return false;
        }
    };
    auto run_from_B = [&](int s) -> bool {
        if (cs != s) return true;
        while (true) {
            load_next(bufA);
            __builtin_amdgcn_sched_barrier(0);
            compute(cs, crow, ct, bufB);
            advance(cs, crow, ct);
            if (cs != s) return false;
            load_next(bufB);
            __builtin_amdgcn_sched_barrier(0);
            compute(cs, crow, ct, bufA);
            advance(cs, crow, ct);
            if (cs != s) return true;
        }
    };

    bool broken = false;     // thread 0 only: a barrier timed out, skip the rest
    bool nextB = false;      // which buffer holds the next step's loads
    for (int s = 0; s < n; ++s) {
        if (s > 0) {
            const ChainStage& st = args.st[s];
            if (st.wait) {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (threadIdx.x == 0 && !broken && !grid_barrier_thread0(args.bar, (unsigned)args.nwg)) broken = true;
                __syncthreads();
                stage_x(s);
            } else if (st.x != args.st[s - 1].x || st.nb != args.st[s - 1].nb) {
                __syncthreads();     // every wave is done with the staged x
                stage_x(s);
            }                        // else: same input, already staged
        }
        nextB = nextB ? run_from_B(s) : run_from_A(s);
    }
}

// Launches one batch of stages.  lds_x: bytes of staged activations (the
// largest stage's); the per-wave weight copies follow them in CONTIG mode.
// The grid is what stays resident (the stage barriers need every
// workgroup running), and no larger than the rows of all stages need.
template <class F, int NW, bool CONTIG>
int32_t launch_chain(ChainArgs& a, size_t lds_x, hipStream_t st) {
    auto kern = chain_kernel<F, NW, CONTIG>;
    const size_t lds = lds_x + (CONTIG ? (size_t)NW * Contig<F>::kStepBytes : 0);
    static size_t dyn_max = 0;   // benign race: every thread computes and sets the same value
    if (!dyn_max) {
        hipFuncAttributes fa;
        if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern)) != hipSuccess)
            return fail(QMV_EHIP, "qmv_chain: cannot query the kernel: %s", hipGetErrorString(hipGetLastError()));
        const size_t m = kLdsMax - fa.sharedSizeBytes;   // the kernel's own __shared__ words come first
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)m) != hipSuccess)
            return fail(QMV_EHIP, "qmv_chain: cannot raise the LDS limit: %s", hipGetErrorString(hipGetLastError()));
        dyn_max = m;
    }
    if (lds > dyn_max) return fail(QMV_EINVAL, "qmv_chain: %zu bytes of staged activations exceed the LDS", lds);
    const int per_cu = resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds);
    int64_t rows = 0;
    for (int s = 0; s < a.n; ++s) rows += a.st[s].N;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((rows + NW - 1) / NW,
                                                                 (int64_t)device_cu_count() * per_cu));
    a.nwg = grid;
    a.xfloats = (int32_t)(lds_x / sizeof(float));
    const int64_t waves = (int64_t)grid * NW;
    int64_t before = 0;
    for (int s = 0; s < a.n; ++s) {
        a.st[s].off = (int32_t)(before % waves);
        before += a.st[s].N;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, a);
    return check_launch("qmv_chain");
}

// Zeroes n words (the chain's barrier words before a call that does not
// rely on an earlier one); a kernel, not a memset, so that it records as a
// kernel node under graph capture.
__global__ __launch_bounds__(256) void zero_words_kernel(unsigned* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// clear: zero the workspace on the stream before the first launch that
// uses its barrier words (qmv_chain_noalloc's library-held copy).
template <class F>
int32_t chain(qmv_fmt fmt, const qmv_chain_stage* stages, int32_t n_stages, void* workspace, size_t ws_bytes,
              void* stream, bool clear = false, const char* name = "qmv_chain") {
    if (!stages || !workspace) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (n_stages < 1) return fail(QMV_EINVAL, "%s: n_stages must be >= 1", name);
    if (ws_bytes < QMV_CHAIN_WORKSPACE_BYTES)
        return fail(QMV_EINVAL, "%s: workspace of %zu bytes < %d", name, ws_bytes, QMV_CHAIN_WORKSPACE_BYTES);
    if (!aligned(workspace, 4)) return fail(QMV_EALIGN, "%s: workspace must be 4-byte aligned", name);
    int max_nb = 0;
    bool contig = true;   // every stage: whole 64-block steps, 16-byte aligned W
    for (int s = 0; s < n_stages; ++s) {
        const qmv_chain_stage& q = stages[s];
        if (!q.W || !q.x || !q.y) return fail(QMV_EINVAL, "%s: stage %d: null pointer", name, s);
        if (q.n_rows < 1 || q.n_rows > (1 << 30))
            return fail(QMV_EINVAL, "%s: stage %d: n_rows must be in 1..2^30", name, s);
        if (q.n_cols < 32 || q.n_cols % 32 || q.n_cols > 35424)
            return fail(QMV_EINVAL, "%s: stage %d: n_cols must be a multiple of 32 in 32..35424", name, s);
        if (!aligned(q.W, 4) || !aligned(q.x, 4) || !aligned(q.y, 4))
            return fail(QMV_EALIGN, "%s: stage %d: W, x and y must be 4-byte aligned", name, s);
        max_nb = std::max(max_nb, (int)(q.n_cols / 32));
        contig = contig && (q.n_cols / 32) % 64 == 0 && aligned(q.W, 16);
    }
    hipStream_t st = as_stream(stream);
    // One group of matvecs on one input (no stage waits, same x and width):
    // the dense contiguous kernel over the stages' concatenated rows, one
    // launch and no stage boundaries (bitwise the same outputs).
    bool group = n_stages <= kMaxSegs;
    for (int s = 1; s < n_stages && group; ++s)
        group = !stages[s].wait && stages[s].x == stages[0].x && stages[s].n_cols == stages[0].n_cols;
    if (group) {
        RowSegs segs = {};
        segs.n = n_stages;
        int64_t rows = 0;
        for (int s = 0; s < n_stages; ++s) {
            segs.W[s] = static_cast<const uint8_t*>(stages[s].W);
            segs.y[s] = stages[s].y;
            rows += stages[s].n_rows;
            segs.end[s] = rows;
        }
        int32_t rc;
        if (group_matvec_contig(fmt, segs, (int)(stages[0].n_cols / 32), stages[0].x, st, true, &rc))
            return rc == QMV_OK ? ok() : rc;
    }
    if (clear) {
        constexpr int words = QMV_CHAIN_WORKSPACE_BYTES / 4;
        hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st,
                           static_cast<unsigned*>(workspace), words);
        if (const int32_t rc = check_launch(name)) return rc;
    }
    {
        // whole 2048-column windows: one weight stream across the levels
        int32_t rc;
        if (decode_chain(fmt, stages, n_stages, static_cast<unsigned*>(workspace), st, &rc))
            return rc == QMV_OK ? ok() : rc;
    }
    const size_t lds_x = (size_t)max_nb * kXPad * sizeof(float);
    const size_t step = Contig<F>::kStepBytes;
    const int contig_nw = !contig ? 0 : lds_x + 8 * step <= (size_t)kLdsMax ? 8
                                      : lds_x + 4 * step <= (size_t)kLdsMax ? 4 : 0;
    for (int s0 = 0; s0 < n_stages; s0 += kChainMaxStages) {
        ChainArgs a = {};
        a.n = std::min(kChainMaxStages, n_stages - s0);
        a.bar = static_cast<unsigned*>(workspace);
        for (int i = 0; i < a.n; ++i) {
            const qmv_chain_stage& q = stages[s0 + i];
            a.st[i].W = static_cast<const uint8_t*>(q.W);
            a.st[i].x = q.x;
            a.st[i].y = q.y;
            a.st[i].N = (int32_t)q.n_rows;
            a.st[i].nb = (int16_t)(q.n_cols / 32);
            a.st[i].wait = (i > 0 && q.wait) ? 1 : 0;   // the first stage of a launch follows a kernel boundary
            a.st[i].xvec = aligned(q.x, 16) ? 1 : 0;
        }
        int32_t rc;
        if (contig_nw == 8) rc = launch_chain<F, 8, true>(a, lds_x, st);
        else if (contig_nw == 4) rc = launch_chain<F, 4, true>(a, lds_x, st);
        else if (lds_x > 40 * 1024) rc = launch_chain<F, 8, false>(a, lds_x, st);
        else rc = launch_chain<F, 4, false>(a, lds_x, st);
        if (rc != QMV_OK) return rc;
    }
    return ok();
}

// Device address of `scratch` on the current device, looked up once per
// device (thread-safe).  QMV_EHIP with a message when the lookup fails.
int32_t scratch_address(void** out) {
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void* addr[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return fail(QMV_EHIP, "qmv_chain_noalloc: no usable current device");
    std::lock_guard<std::mutex> g(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(QMV_EHIP, "qmv_chain_noalloc: cannot find the library's barrier words: %s",
                        hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return QMV_OK;
}

}  // namespace
}  // namespace qmv

extern "C" int32_t qmv_chain(qmv_fmt fmt, const qmv_chain_stage* stages, int32_t n_stages, void* workspace,
                             size_t workspace_bytes, void* stream) {
    switch (fmt) {
    case QMV_Q8_0: return qmv::chain<qmv::Q8_0>(fmt, stages, n_stages, workspace, workspace_bytes, stream);
    case QMV_Q4_0: return qmv::chain<qmv::Q4_0>(fmt, stages, n_stages, workspace, workspace_bytes, stream);
    case QMV_Q4_1: return qmv::chain<qmv::Q4_1>(fmt, stages, n_stages, workspace, workspace_bytes, stream);
    default: {
        const qmv::FormatOps* ops = qmv::format_ops(fmt);
        if (!ops || !ops->chain) return qmv::fail(QMV_EUNSUPPORTED, "qmv_chain: unknown format %d", (int)fmt);
        if (!workspace) return qmv::fail(QMV_EINVAL, "qmv_chain: null pointer");
        if (workspace_bytes < QMV_CHAIN_WORKSPACE_BYTES)
            return qmv::fail(QMV_EINVAL, "qmv_chain: workspace of %zu bytes < %d", workspace_bytes,
                             QMV_CHAIN_WORKSPACE_BYTES);
        return ops->chain("qmv_chain", stages, n_stages, stream);
    }
    }
}

extern "C" int32_t qmv_chain_noalloc(qmv_fmt fmt, const qmv_chain_stage* stages, int32_t n_stages, void* stream) {
    const char* name = "qmv_chain_noalloc";
    void* ws = nullptr;
    if (fmt != QMV_Q8_0 && fmt != QMV_Q4_0 && fmt != QMV_Q4_1) {
        // no barrier words: the stages run as separate launches
        const qmv::FormatOps* ops = qmv::format_ops(fmt);
        if (!ops || !ops->chain) return qmv::fail(QMV_EUNSUPPORTED, "%s: unknown format %d", name, (int)fmt);
        return ops->chain(name, stages, n_stages, stream);
    }
    if (!stages) return qmv::fail(QMV_EINVAL, "%s: null pointer", name);
    if (n_stages < 1) return qmv::fail(QMV_EINVAL, "%s: n_stages must be >= 1", name);
    if (const int32_t rc = qmv::scratch_address(&ws)) return rc;
    switch (fmt) {
    case QMV_Q8_0: return qmv::chain<qmv::Q8_0>(fmt, stages, n_stages, ws, QMV_CHAIN_WORKSPACE_BYTES, stream, true, name);
    case QMV_Q4_0: return qmv::chain<qmv::Q4_0>(fmt, stages, n_stages, ws, QMV_CHAIN_WORKSPACE_BYTES, stream, true, name);
    default: return qmv::chain<qmv::Q4_1>(fmt, stages, n_stages, ws, QMV_CHAIN_WORKSPACE_BYTES, stream, true, name);
    }
}
