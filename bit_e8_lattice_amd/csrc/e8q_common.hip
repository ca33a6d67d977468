// Host-only entry points and shared host state.
#include <atomic>
#include <mutex>

#include "e8q_core_table.hpp"
#include "e8q_host.hpp"

namespace e8q {

int64_t core_size_host(int32_t bound);

int device_cu_count() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev >= 64) dev = 63;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] <= 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
            cu = 256;
        cache[dev] = cu;
    }
    return cache[dev];
}

}  // namespace e8q

extern "C" int64_t e8q_core_size(int32_t core_bound) {
    if (core_bound < 0 || core_bound > 40) return -1;
    return e8q::core_size_host(core_bound);
}

extern "C" const char* e8q_status_string(e8q_status_t s) {
    switch (s) {
        case E8Q_OK: return "ok";
        case E8Q_ERR_INVALID: return "invalid argument";
        case E8Q_ERR_UNSUPPORTED: return "unsupported dtype or size";
        case E8Q_ERR_LAUNCH: return "kernel launch failed";
        case E8Q_ERR_DEVICE: return "device query or table upload failed";
        default: return "unknown status";
    }
}

extern "C" const char* e8q_version(void) { return "e8q 0.1.0 gfx950"; }
