// All-integer int8 matrix x vector product with per-output-channel requant,
// for gfx950.
//
// What is computed ("Blue -- porting zen-nano (Qwen3-0.6B) to deterministic
// on-chain inference", "Quantization recipe"): int8 weights and
// activations, int32 accumulation, then per output channel
//   y = sat_int8(RoundingDivideByPOT(SaturatingRoundingDoublingHighMul(acc,
//       mult[o]), shift[o])).
// The page names the two gemmlowp functions only; the readings used here
// are: SRDHM(a, m) = a*m / 2^31 rounded to nearest with ties toward
// +infinity (saturating the single overflow case -2^31 * -2^31), and
// RDBPOT(v, e) = v / 2^e rounded to nearest with ties away from zero.
//
// The same page's integer engine runs its activation functions (SiLU among
// them) as frozen lookup tables; qmv_i8_requant_lut applies such a table to
// the requantized output in the epilogue: y = lut[y + 128].
//
// Mapping: rows are split into segments of LPR lanes; each lane reads
// 16 consecutive weight bytes per step (one 16-byte load; a segment reads
// 16*LPR contiguous bytes), multiplies them with the matching 16 activation
// bytes by four v_dot4_i32_i8, and the segment sums its lanes' int32
// partials exactly.  The epilogue runs in one lane per row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "qmv_host.h"

namespace qmv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 ld16_nt(const int8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}
__device__ __forceinline__ i32x4 ld16(const int8_t* p) { return *reinterpret_cast<const i32x4*>(p); }

// a*m / 2^31, nearest, ties toward +inf: the arithmetic shift of
// a*m + 2^30 by 31 is floor((a*m + 2^30) / 2^31).
__device__ __forceinline__ int32_t srdhm(int32_t a, int32_t m) {
    if (a == INT_MIN && m == INT_MIN) return INT_MAX;
    const int64_t p = (int64_t)a * (int64_t)m;
    return (int32_t)((p + ((int64_t)1 << 30)) >> 31);
}

// v / 2^e, nearest, ties away from zero: floor division plus one when the
// remainder exceeds half the divisor (half included for negative v).
__device__ __forceinline__ int32_t rdbpot(int32_t v, int32_t e) {
    e = e < 0 ? 0 : (e > 31 ? 31 : e);   // out-of-contract shifts stay defined
    const int64_t mask = ((int64_t)1 << e) - 1;
    const int64_t rem = (int64_t)v & mask;
    const int64_t thr = (mask >> 1) + (v < 0 ? 1 : 0);
    return (int32_t)(((int64_t)v >> e) + (rem > thr ? 1 : 0));
}

__device__ __forceinline__ int8_t sat8(int32_t v) { return (int8_t)(v < -128 ? -128 : (v > 127 ? 127 : v)); }

// Exact int32 sum over the LPR consecutive lanes of a segment; valid in the
// segment's first lane.  DPP swizzles within 16-lane rows, scalar reads
// across rows.
template <int CTRL>
__device__ __forceinline__ int32_t dpp_mov(int32_t v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int LPR>
__device__ __forceinline__ int32_t segment_sum(int32_t v) {
    static_assert(LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "segment width");
    v += dpp_mov<0xB1>(v);     // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);     // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);    // row_half_mirror
    if (LPR >= 16) v += dpp_mov<0x140>(v);   // row_mirror
    if (LPR == 32) {
        const int32_t a = __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16);
        const int32_t b = __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
        v = (threadIdx.x & 32) ? b : a;
    } else if (LPR == 64) {
        v = __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
            __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
    }
    return v;
}

template <int B, int LPR, int RPL>
__global__ __launch_bounds__(kThreads) void i8_kernel(const int8_t* __restrict__ W, int64_t N, int nc,
                                                      const int8_t* __restrict__ x, int64_t ldx,
                                                      const int32_t* __restrict__ mult,
                                                      const int32_t* __restrict__ shift,
                                                      const int8_t* __restrict__ lut, int8_t* __restrict__ y,
                                                      int64_t ldy) {
    constexpr int G = 64 / LPR;
    constexpr int ROWS = G * RPL;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int seg = lane / LPR;
    const int li = lane % LPR;
    const int64_t K = (int64_t)nc * 16;

    for (int64_t tile = (int64_t)blockIdx.x * kWaves + wave; tile * ROWS < N; tile += (int64_t)gridDim.x * kWaves) {
        const int64_t row0 = tile * ROWS;
        const int8_t* wr[RPL];
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int64_t row = row0 + r * G + seg;
            wr[r] = W + (row < N ? row : N - 1) * K;
        }
        int32_t acc[RPL][B];
#pragma unroll
        for (int r = 0; r < RPL; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = 0;

        for (int c = li; c < nc; c += LPR) {
            i32x4 w[RPL];
#pragma unroll
            for (int r = 0; r < RPL; ++r) w[r] = ld16_nt(wr[r] + 16 * c);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const i32x4 xv = ld16(x + b * ldx + 16 * c);
#pragma unroll
                for (int r = 0; r < RPL; ++r) {
                    int32_t a = acc[r][b];
                    a = __builtin_amdgcn_sdot4(w[r].x, xv.x, a, false);
                    a = __builtin_amdgcn_sdot4(w[r].y, xv.y, a, false);
                    a = __builtin_amdgcn_sdot4(w[r].z, xv.z, a, false);
                    a = __builtin_amdgcn_sdot4(w[r].w, xv.w, a, false);
                    acc[r][b] = a;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RPL; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = segment_sum<LPR>(acc[r][b]);
        if (li == 0) {
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int64_t row = row0 + r * G + seg;
                if (row < N) {
                    const int32_t mu = mult[row], sh = shift[row];
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const int8_t v = sat8(rdbpot(srdhm(acc[r][b], mu), sh));
                        y[b * ldy + row] = lut ? lut[v + 128] : v;   // lut: a kernel argument, uniform
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- pipelined form
// Rows of whole 1024-byte steps (n_cols a multiple of 1024, as every
// Qwen3-0.6B shape): a wave streams row groups of RR rows with the next
// pipeline slot's loads in flight while one is computed, across row
// groups.  Lane l loads bytes 16 l .. 16 l + 15 of each 1024-byte step
// through a per-row buffer descriptor (scalar row base, lane-constant
// offset).  Activations either sit in registers for the whole launch (TX >
// 0: rows of TX steps at batch B with B TX <= 8; a slot then holds all TX
// steps of the group's rows) or are staged once per workgroup in LDS (TX ==
// 0: a slot holds one step of each row).  Each slot also carries the mult
// and shift of the lane's epilogue row, read with the weights through
// buffer descriptors (rows past the end read 0 and are not stored), so the
// epilogue waits on no memory access of its own.  The table of the _lut
// form sits in registers (lane l holds entries 4 l .. 4 l + 3) and is
// looked up across lanes.  The epilogue of a row group runs in RR x B lanes
// at once (lane k + RR b: row k of the group, column b).  Sums are exact
// int32, so every output equals i8_kernel's.
constexpr int kI8Step = 1024;
constexpr int kBufNT = 2;   // buffer-load cache policy: non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t i8_buffer(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);   // raw buffer
}

template <int RR, int SW>
struct I8Slot {
    i32x4 w[RR][SW];
    int32_t m, s;
};

template <int B, int RR, int NW, int TX>
__global__ __launch_bounds__(64 * NW) void i8_stream_kernel(const int8_t* __restrict__ W, int N, int T_arg,
                                                             const int8_t* __restrict__ x, int64_t ldx,
                                                             const int32_t* __restrict__ mult,
                                                             const int32_t* __restrict__ shift,
                                                             const int8_t* __restrict__ lut, int8_t* __restrict__ y,
                                                             int64_t ldy) {
    static_assert(RR * B <= 64 && (RR & (RR - 1)) == 0, "epilogue lanes");
    static_assert(TX == 0 || B * TX <= 8, "activations held in registers");
    constexpr int SW = TX > 0 ? TX : 1;             // steps of a row per slot
    extern __shared__ __attribute__((aligned(16))) i32x4 xs[];   // TX == 0: [B][T * 64] chunks of 16 bytes
    const int T = TX > 0 ? TX : T_arg;              // steps per row
    const int TS = TX > 0 ? 1 : T;                  // slots per row group
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t K = (uint32_t)T * kI8Step;
    const int NP = (N + RR - 1) / RR;
    const int wstride = (int)gridDim.x * NW;
    const int ek = lane % RR, eb = lane / RR;
    const __amdgpu_buffer_rsrc_t mrs = i8_buffer(mult, 4u * (uint32_t)N);
    const __amdgpu_buffer_rsrc_t srs = i8_buffer(shift, 4u * (uint32_t)N);

    int32_t lutw = 0;
    if (lut)
        lutw = (int32_t)((uint32_t)(uint8_t)lut[4 * lane] | (uint32_t)(uint8_t)lut[4 * lane + 1] << 8 |
                         (uint32_t)(uint8_t)lut[4 * lane + 2] << 16 | (uint32_t)(uint8_t)lut[4 * lane + 3] << 24);

    int lrow = (int)blockIdx.x * NW + wave, lt = 0;   // load cursor: row group, slot
    int crow = lrow, ct = 0;                          // compute cursor
    __amdgpu_buffer_rsrc_t lrs[RR];
    auto set_rows = [&](int p) {
#pragma unroll
        for (int k = 0; k < RR; ++k) lrs[k] = i8_buffer(W + (int64_t)min(RR * p + k, N - 1) * K, K);
    };
    set_rows(min(lrow, NP - 1));
    // Called while the load cursor is inside the wave's rows, and once at
    // the start by waves without rows (their loads stay inside W through the
    // clamped descriptors, and mult / shift past the end read 0).
    auto load_next = [&](I8Slot<RR, SW>& sl) {
        const int t = lt;
        const int g = lrow;
#pragma unroll
        for (int k = 0; k < RR; ++k)
#pragma unroll
            for (int u = 0; u < SW; ++u) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(lrs[k], 16 * lane, (t * SW + u) * kI8Step, kBufNT);
                sl.w[k][u] = i32x4{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
            }
        const int goff = (int)(4u * RR * (uint32_t)g);   // < 2^32 bytes: a byte offset into mult / shift
        sl.m = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(mrs, 4 * ek, goff, 0);
        sl.s = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(srs, 4 * ek, goff, 0);
        if (++lt == TS) {
            lt = 0;
            lrow += wstride;
            set_rows(min(lrow, NP - 1));
        }
    };
    i32x4 xr[B][SW];   // TX > 0: the lane's activation chunks
    int32_t acc[RR][B];
#pragma unroll
    for (int k = 0; k < RR; ++k)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[k][b] = 0;
    auto compute = [&](const I8Slot<RR, SW>& sl, int t) {
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int u = 0; u < SW; ++u) {
                const i32x4 xv = TX > 0 ? xr[b][u] : xs[(b * T + t) * 64 + lane];
#pragma unroll
                for (int k = 0; k < RR; ++k) {
                    int32_t a = acc[k][b];
                    a = __builtin_amdgcn_sdot4(sl.w[k][u].x, xv.x, a, false);
                    a = __builtin_amdgcn_sdot4(sl.w[k][u].y, xv.y, a, false);
                    a = __builtin_amdgcn_sdot4(sl.w[k][u].z, xv.z, a, false);
                    a = __builtin_amdgcn_sdot4(sl.w[k][u].w, xv.w, a, false);
                    acc[k][b] = a;
                }
            }
        if (t == TS - 1) {
            int32_t mine = 0;
#pragma unroll
            for (int k = 0; k < RR; ++k)
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int32_t tot = segment_sum<64>(acc[k][b]);
                    if (k == ek && b == eb) mine = tot;
                    acc[k][b] = 0;
                }
            int32_t v = sat8(rdbpot(srdhm(mine, sl.m), sl.s));
            if (lut) {   // every lane takes part in the cross-lane read
                const int idx = v + 128;
                const int32_t wv = __builtin_amdgcn_ds_bpermute((idx >> 2) << 2, lutw);
                v = (int8_t)(wv >> (8 * (idx & 3)));
            }
            const int row = RR * crow + ek;
            if (eb < B && row < N) y[eb * ldy + row] = (int8_t)v;
        }
    };

    // Activation loads go out before the first weight loads; with staging
    // of one chunk per thread the store then waits for that chunk only
    // (loads complete in order).
    I8Slot<RR, SW> s0, s1;
    const int nch = B * T * 64;
    if constexpr (TX > 0) {
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int u = 0; u < TX; ++u) xr[b][u] = ld16(x + b * ldx + u * kI8Step + 16 * lane);
        load_next(s0);
    } else {
        if (nch <= 64 * NW) {
            const int i = threadIdx.x;
            i32x4 xv = {0, 0, 0, 0};
            if (i < nch) xv = ld16(x + (i / (T * 64)) * ldx + 16 * (i % (T * 64)));
            load_next(s0);
            __builtin_amdgcn_sched_barrier(0);
            if (i < nch) xs[i] = xv;
        } else {
            for (int i = threadIdx.x; i < nch; i += 64 * NW)
                xs[i] = ld16(x + (i / (T * 64)) * ldx + 16 * (i % (T * 64)));
            load_next(s0);
        }
        __syncthreads();
    }

    auto advance = [&]() {
        if (++ct == TS) {
            ct = 0;
            crow += wstride;
        }
    };
    // The load cursor runs one slot ahead; once it is past the wave's last
    // slot, the slot in hand is the last one and nothing more is loaded.
    if (crow < NP) {
        while (true) {
            if (lrow >= NP) {
                compute(s0, ct);
                break;
            }
            load_next(s1);
            __builtin_amdgcn_sched_barrier(0);
            compute(s0, ct);
            advance();
            if (lrow >= NP) {
                compute(s1, ct);
                break;
            }
            load_next(s0);
            __builtin_amdgcn_sched_barrier(0);
            compute(s1, ct);
            advance();
        }
    }
}

// Largest activation block (batch x n_cols bytes) the pipelined form stages.
constexpr int64_t kI8StreamLds = 32768;

template <int B, int RR, int NW, int TX = 0>
int32_t launch_stream(const int8_t* W, int64_t N, int64_t K, const int8_t* x, int64_t ldx, const int32_t* mult,
                      const int32_t* shift, const int8_t* lut, int8_t* y, int64_t ldy, hipStream_t st) {
    auto kern = i8_stream_kernel<B, RR, NW, TX>;
    const size_t lds = TX > 0 ? 0 : (size_t)B * (size_t)K;
    const int64_t tiles = ((N + RR - 1) / RR + NW - 1) / NW;
    const int per_cu = std::max(1, resident_wgs(reinterpret_cast<const void*>(kern), 64 * NW, lds));
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, (int64_t)device_cu_count() * per_cu));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, W, (int)N, (int)(K / kI8Step), x, ldx, mult, shift,
                       lut, y, ldy);
    return check_launch("qmv_i8_requant");
}

// Four rows per group and 8 waves on tall matrices (the lm_head).  Shorter
// ones at batch 1 with rows of up to 4 steps keep the activations in
// registers (no staging, no barrier: these launches are latency-bound),
// two rows per group; otherwise one row per group and 4 waves.
template <int B>
int32_t launch_stream_rows(const int8_t* W, int64_t N, int64_t K, const int8_t* x, int64_t ldx, const int32_t* mult,
                           const int32_t* shift, const int8_t* lut, int8_t* y, int64_t ldy, hipStream_t st) {
    if (N >= 16384) return launch_stream<B, 4, 8>(W, N, K, x, ldx, mult, shift, lut, y, ldy, st);
    if constexpr (B == 1) {
        switch (K / kI8Step) {
        case 1: return launch_stream<1, 2, 4, 1>(W, N, K, x, ldx, mult, shift, lut, y, ldy, st);
        case 2: return launch_stream<1, 2, 4, 2>(W, N, K, x, ldx, mult, shift, lut, y, ldy, st);
        case 3: return launch_stream<1, 2, 4, 3>(W, N, K, x, ldx, mult, shift, lut, y, ldy, st);
        case 4: return launch_stream<1, 2, 4, 4>(W, N, K, x, ldx, mult, shift, lut, y, ldy, st);
        default: break;
        }
    }
    return launch_stream<B, 1, 4>(W, N, K, x, ldx, mult, shift, lut, y, ldy, st);
}

constexpr int kRpl = 2;

template <int B, int LPR>
int32_t launch_b(const int8_t* W, int64_t N, int nc, const int8_t* x, int64_t ldx, const int32_t* mult,
                 const int32_t* shift, const int8_t* lut, int8_t* y, int64_t ldy, hipStream_t st) {
    constexpr int rows_per_wg = kWaves * (64 / LPR) * kRpl;
    const int64_t tiles = (N + rows_per_wg - 1) / rows_per_wg;
    const int grid = (int)std::min<int64_t>(tiles, (int64_t)device_cu_count() * 8);
    hipLaunchKernelGGL((i8_kernel<B, LPR, kRpl>), dim3(grid), dim3(kThreads), 0, st, W, N, nc, x, ldx, mult, shift,
                       lut, y, ldy);
    return check_launch("qmv_i8_requant");
}

template <int B>
int32_t launch_lpr(const int8_t* W, int64_t N, int nc, const int8_t* x, int64_t ldx, const int32_t* mult,
                   const int32_t* shift, const int8_t* lut, int8_t* y, int64_t ldy, hipStream_t st) {
    if (nc >= 64) return launch_b<B, 64>(W, N, nc, x, ldx, mult, shift, lut, y, ldy, st);
    if (nc >= 32) return launch_b<B, 32>(W, N, nc, x, ldx, mult, shift, lut, y, ldy, st);
    return launch_b<B, 8>(W, N, nc, x, ldx, mult, shift, lut, y, ldy, st);
}

int32_t i8_requant(const char* name, const int8_t* W, int64_t n_rows, int64_t n_cols, const int8_t* x, int64_t ldx,
                   int32_t batch, const int32_t* mult, const int32_t* shift, const int8_t* lut, int8_t* y,
                   int64_t ldy, void* stream) {
    if (!W || !x || !mult || !shift || !y) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (n_rows < 1) return fail(QMV_EINVAL, "%s: n_rows must be >= 1 (got %lld)", name, (long long)n_rows);
    if (n_cols < 16 || n_cols % 16 || n_cols > 131056)
        return fail(QMV_EINVAL, "%s: n_cols must be a multiple of 16 in 16..131056 (got %lld)", name,
                    (long long)n_cols);
    if (batch < 1 || batch > 8) return fail(QMV_EINVAL, "%s: batch must be in 1..8 (got %d)", name, batch);
    if (ldx < n_cols) return fail(QMV_EINVAL, "%s: ldx (%lld) < n_cols (%lld)", name, (long long)ldx, (long long)n_cols);
    if (ldy < n_rows) return fail(QMV_EINVAL, "%s: ldy (%lld) < n_rows (%lld)", name, (long long)ldy, (long long)n_rows);
    if (n_rows > ((int64_t)1 << 40) / n_cols) return fail(QMV_EINVAL, "%s: matrix too large", name);
    if (!aligned(W, 16) || !aligned(x, 16) || ldx % 16)
        return fail(QMV_EALIGN, "%s: W and x must be 16-byte aligned and ldx a multiple of 16", name);
    if (!aligned(mult, 4) || !aligned(shift, 4)) return fail(QMV_EALIGN, "%s: mult/shift must be 4-byte aligned", name);
    const int nc = (int)(n_cols / 16);
    hipStream_t st = as_stream(stream);
    if (n_cols % kI8Step == 0 && batch * n_cols <= kI8StreamLds) {
        switch (batch) {
        case 1: return launch_stream_rows<1>(W, n_rows, n_cols, x, ldx, mult, shift, lut, y, ldy, st);
        case 2: return launch_stream_rows<2>(W, n_rows, n_cols, x, ldx, mult, shift, lut, y, ldy, st);
        case 3: return launch_stream_rows<3>(W, n_rows, n_cols, x, ldx, mult, shift, lut, y, ldy, st);
        case 4: return launch_stream_rows<4>(W, n_rows, n_cols, x, ldx, mult, shift, lut, y, ldy, st);
        case 5: return launch_stream_rows<5>(W, n_rows, n_cols, x, ldx, mult, shift, lut, y, ldy, st);
        case 6: return launch_stream_rows<6>(W, n_rows, n_cols, x, ldx, mult, shift, lut, y, ldy, st);
        case 7: return launch_stream_rows<7>(W, n_rows, n_cols, x, ldx, mult, shift, lut, y, ldy, st);
        default: return launch_stream_rows<8>(W, n_rows, n_cols, x, ldx, mult, shift, lut, y, ldy, st);
        }
    }
    switch (batch) {
    case 1: return launch_lpr<1>(W, n_rows, nc, x, ldx, mult, shift, lut, y, ldy, st);
    case 2: return launch_lpr<2>(W, n_rows, nc, x, ldx, mult, shift, lut, y, ldy, st);
    case 3: return launch_lpr<3>(W, n_rows, nc, x, ldx, mult, shift, lut, y, ldy, st);
    case 4: return launch_lpr<4>(W, n_rows, nc, x, ldx, mult, shift, lut, y, ldy, st);
    case 5: return launch_lpr<5>(W, n_rows, nc, x, ldx, mult, shift, lut, y, ldy, st);
    case 6: return launch_lpr<6>(W, n_rows, nc, x, ldx, mult, shift, lut, y, ldy, st);
    case 7: return launch_lpr<7>(W, n_rows, nc, x, ldx, mult, shift, lut, y, ldy, st);
    default: return launch_lpr<8>(W, n_rows, nc, x, ldx, mult, shift, lut, y, ldy, st);
    }
}

}  // namespace
}  // namespace qmv

extern "C" int32_t qmv_i8_requant(const int8_t* W, int64_t n_rows, int64_t n_cols, const int8_t* x, int64_t ldx,
                                  int32_t batch, const int32_t* mult, const int32_t* shift, int8_t* y, int64_t ldy,
                                  void* stream) {
    return qmv::i8_requant("qmv_i8_requant", W, n_rows, n_cols, x, ldx, batch, mult, shift, nullptr, y, ldy, stream);
}

extern "C" int32_t qmv_i8_requant_lut(const int8_t* W, int64_t n_rows, int64_t n_cols, const int8_t* x, int64_t ldx,
                                      int32_t batch, const int32_t* mult, const int32_t* shift, const int8_t* lut,
                                      int8_t* y, int64_t ldy, void* stream) {
    if (!lut) return qmv::fail(QMV_EINVAL, "qmv_i8_requant_lut: null table");
    return qmv::i8_requant("qmv_i8_requant_lut", W, n_rows, n_cols, x, ldx, batch, mult, shift, lut, y, ldy, stream);
}
