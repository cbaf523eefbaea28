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
