// Host-side helpers of libqmv.so (see qmv_host.h).
#include "qmv_host.h"

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

namespace qmv {

namespace {
thread_local char g_err[512] = {0};
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
}  // namespace

int32_t fail(int32_t code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int32_t ok() {
    g_err[0] = 0;
    return QMV_OK;
}

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

int resident_wgs(const void* kernel, int threads, size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<const void*, size_t>, int> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const auto key = std::make_pair(kernel, lds * 64 + (size_t)dev);
    {
        std::lock_guard<std::mutex> g(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        n = 1;
    }
    std::lock_guard<std::mutex> g(mu);
    cache[key] = n;
    return n;
}

int32_t lds_limit(const void* kernel, size_t lds_total, const char* what, size_t* dyn_max) {
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, size_t> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(QMV_EHIP, "%s: no current device: %s", what, hipGetErrorString(hipGetLastError()));
    const auto key = std::make_pair(kernel, dev);
    std::lock_guard<std::mutex> g(mu);
    auto it = done.find(key);
    if (it != done.end()) {
        *dyn_max = it->second;
        return QMV_OK;
    }
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, kernel) != hipSuccess)
        return fail(QMV_EHIP, "%s: cannot query the kernel: %s", what, hipGetErrorString(hipGetLastError()));
    if (fa.sharedSizeBytes >= lds_total) return fail(QMV_EHIP, "%s: the kernel's static LDS fills the workgroup", what);
    const size_t m = lds_total - fa.sharedSizeBytes;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)m) != hipSuccess)
        return fail(QMV_EHIP, "%s: cannot raise the LDS limit: %s", what, hipGetErrorString(hipGetLastError()));
    done[key] = m;
    *dyn_max = m;
    return QMV_OK;
}

int32_t check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QMV_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace qmv

extern "C" const char* qmv_last_error(void) { return qmv::g_err; }
extern "C" int32_t qmv_abi_version(void) { return QMV_ABI_VERSION; }
