// Host-only entry points and shared host state.
#include <cstddef>
#include <mutex>

#include "e8q_host.hpp"
#include "e8q_tables_index.h"

// The record layouts are part of the ABI (kernels read and write them as
// 32-bit words).
static_assert(sizeof(e8q_escape_t) == 20 && alignof(e8q_escape_t) == 4, "escape record layout");
static_assert(offsetof(e8q_escape_t, two_z) == 4, "escape record layout");
static_assert(sizeof(e8q_escape_packed_t) == 8, "packed record layout");
static_assert(offsetof(e8q_escape_packed_t, core_idx) == 4 && offsetof(e8q_escape_packed_t, root) == 6,
              "packed record layout");

namespace e8q {

const unsigned char* table_blob_address();

const DevTable* get_table(int32_t bound, e8q_status_t& err) {
    if (bound < 0 || bound > 40) {
        err = E8Q_ERR_INVALID;
        return nullptr;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        err = E8Q_ERR_DEVICE;
        return nullptr;
    }
    static std::mutex mu;
    static DevTable tabs[64][kCanonBounds];
    static bool ready[64][kCanonBounds] = {};
    const int c = bound / 8;   // C(B) = C(8 * floor(B / 8)): ||2z||^2 is a multiple of 8 on E8
    std::lock_guard<std::mutex> lk(mu);
    if (!ready[dev][c]) {
        const unsigned char* base = table_blob_address();
        if (!base) {
            err = E8Q_ERR_DEVICE;
            return nullptr;
        }
        const TableSetLayout& L = gen::kSets[c];
        DevTable& t = tabs[dev][c];
        t.dptr = reinterpret_cast<const uint16_t*>(base + L.rank);
        t.dpoints = reinterpret_cast<const uint32_t*>(base + L.points);
        t.droots = reinterpret_cast<const uint32_t*>(base + gen::kRootsOffset);
        t.dpts64 = reinterpret_cast<const double*>(base + L.p64);
        t.dtiles = base + L.tiles;
        t.ntiles = L.ntiles;
        t.dpts_bf16 = reinterpret_cast<const uint4*>(base + L.pbf);
        t.dh8 = reinterpret_cast<const uint32_t*>(base + L.h8);
        t.p = L.p;
        t.size = L.size;
        ready[dev][c] = true;
    }
    return &tabs[dev][c];
}

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
    return e8q::gen::kSets[core_bound / 8].size;
}

extern "C" const char* e8q_status_string(e8q_status_t s) {
    switch (s) {
        case E8Q_OK: return "ok";
        case E8Q_ERR_INVALID: return "invalid argument";
        case E8Q_ERR_UNSUPPORTED: return "unsupported dtype or size";
        case E8Q_ERR_LAUNCH: return "kernel launch failed";
        case E8Q_ERR_DEVICE: return "device query failed";
        case E8Q_ERR_SCRATCH: return "input too large for the allocation-free entry point's fixed scratch";
        default: return "unknown status";
    }
}

extern "C" const char* e8q_version(void) { return "e8q 0.1.0 gfx950"; }
