// Stream-read ceiling of the device: a buffer read once with 16-byte
// non-temporal loads (the load form of the whole-line matvec kernel), with
// no arithmetic beyond keeping the loads live.  It is the measured
// denominator beside the spec peak.  "Economical Serving and the hanzo.ai
// Platform", Sec. 2.1, sets a standalone read microbenchmark's achievable
// bandwidth beside the spec figure, and "One Native Stack for Private,
// Continuously-Learning AI", "Honest Risks", states which denominator each
// efficiency claim uses; the matvec kernels here are reported against both.
//
// Each lane XORs every 32-bit word it reads and writes one word, so the
// XOR of all output words equals the XOR of the whole buffer: an exact
// check that every byte was read once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "qmv_host.h"

namespace qmv {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;

__device__ __forceinline__ unsigned fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Workgroup b reads the contiguous chunk [b * per, (b + 1) * per) of
// 16-byte vectors, 256 threads side by side, 8 loads in flight per thread.
// Measured on a 4 GiB buffer (7 launches each): this form 6.9-7.0 TB/s;
// a grid-stride loop with four loads 8 MB apart 5.6-6.2 TB/s.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                                     int64_t per, unsigned* __restrict__ out) {
    constexpr int U = 8;
    const int64_t s = min(n16, (int64_t)blockIdx.x * per);
    const int64_t e = min(n16, s + per);
    unsigned acc = 0;
    int64_t i = s + threadIdx.x;
    for (; i + (U - 1) * kStreamThreads < e; i += U * kStreamThreads) {   // every index < e <= n16
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(p + i + k * kStreamThreads);
#pragma unroll
        for (int k = 0; k < U; ++k) acc ^= fold(v[k]);
    }
    for (; i < e; i += kStreamThreads) acc ^= fold(__builtin_nontemporal_load(p + i));
    out[(int64_t)blockIdx.x * kStreamThreads + threadIdx.x] = acc;
}

}  // namespace
}  // namespace qmv

extern "C" int32_t qmv_stream_read(const void* buf, size_t bytes, uint32_t* out, size_t out_words, void* stream) {
    using namespace qmv;
    const char* name = "qmv_stream_read";
    if (!buf || !out) return fail(QMV_EINVAL, "%s: null pointer", name);
    if (bytes < 16 || bytes % 16) return fail(QMV_EINVAL, "%s: bytes must be a positive multiple of 16", name);
    if (out_words < (size_t)kStreamThreads)
        return fail(QMV_EINVAL, "%s: out_words must be >= %d (got %zu)", name, kStreamThreads, out_words);
    if (!aligned(buf, 16) || !aligned(out, 4)) return fail(QMV_EALIGN, "%s: buf 16-byte, out 4-byte aligned", name);
    const int64_t n16 = (int64_t)(bytes / 16);
    // 4 workgroups of 4 waves per CU (measured best of 4, 8 and 16 per CU),
    // no more than the output holds or the buffer needs; chunks are whole
    // multiples of one 8-load round
    const int64_t grid = std::max<int64_t>(
        1, std::min<int64_t>({(int64_t)device_cu_count() * 4, (int64_t)(out_words / kStreamThreads),
                              (n16 + kStreamThreads - 1) / kStreamThreads}));
    constexpr int64_t kRound = 8 * kStreamThreads;
    const int64_t per = ((n16 + grid - 1) / grid + kRound - 1) / kRound * kRound;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kStreamThreads), 0, as_stream(stream),
                       static_cast<const u32x4*>(buf), n16, per, out);
    return check_launch(name);
}
