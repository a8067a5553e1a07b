// rq_device.cpp -- per-device launch facts shared by the kernel launchers:
// the compute-unit count and the dynamic-LDS limit of a kernel.  Both are
// cached per device and safe to use from several host threads at once.

#include <hip/hip_runtime.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "rq_internal.h"

namespace rq {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];   // 0: not read yet

std::mutex g_lds_mu;
std::map<std::pair<const void *, int>, size_t> g_lds_limit;   // (kernel, device) -> bytes set
}  // namespace

int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    return dev;
}

int device_cus() {
    const int dev = current_device();
    if (dev >= kMaxDevices) {
        int n = 0;
        return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0
                   ? n
                   : 256;
    }
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

int ensure_dyn_lds(const void *kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return (int)hipSuccess;
    const int dev = current_device();
    std::lock_guard<std::mutex> lock(g_lds_mu);
    size_t &set = g_lds_limit[std::make_pair(kernel, dev)];
    if (bytes <= set) return (int)hipSuccess;
    const hipError_t e =
        hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) set = bytes;
    return (int)e;
}

}  // namespace rq
