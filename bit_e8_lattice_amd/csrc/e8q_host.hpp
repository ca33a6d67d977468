// Host-side helpers shared by the entry points: argument checks, device
// properties, launch sizing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

#include "e8q.h"
#include "e8q_core_table.hpp"
#include "e8q_tables_build.hpp"

namespace e8q {

// Core tables of one core bound on one device: pointers into the table blob
// that the device code object carries (built with the library, see
// e8q_tables_build.hpp), and the host-side rank parameters.
struct DevTable {
    const uint16_t* dptr = nullptr;      // rank table
    const uint32_t* dpoints = nullptr;   // points in rank order, two words each (2z + 64 bytes)
    const uint32_t* droots = nullptr;    // the 240 roots (same word layout as the points)
    const double* dpts64 = nullptr;      // points in rank order as 9 doubles: t_0..t_7 (= 2z), ||t||^2 / 4
    // The points grouped by norm shell into tiles of 32 rows for the
    // matrix-core search, one of each pair +-t (first nonzero coordinate
    // positive; the origin alone); a shell's last tile is padded with zero
    // rows, and an odd tile count gets one more tile of pads with norm 1e30
    // (its key is never the best).  Per tile, at these offsets (in tiles of
    // ntiles):
    //   0            : 32 rows x 8 bf16 (t = 2z)            512 B per tile
    //   ntiles * 512 : 32 rows x 8 int8 (t)                 256 B per tile
    //   ntiles * 768 : 32 uint16 core indices of t (pads: the origin's)  64 B
    //   ntiles * 832 : 32 uint16 core indices of -t (pads: the origin's) 64 B
    //   ntiles * 896 : the shell's ||t||^2 / 4 as float        4 B per tile
    const uint8_t* dtiles = nullptr;
    uint32_t ntiles = 0;
    // The points in rank order as 8 bfloat16 (2z) each, plus a zero entry at
    // index |C(B)| (the GEMV's matrix-core operand table).
    const uint4* dpts_bf16 = nullptr;
    // H_8 (2z) of every point (natural-order 8-point Walsh-Hadamard transform,
    // exact in integers, |entry| <= 48 for any supported core) as signed bytes,
    // two words per point in the layout of the points.
    const uint32_t* dh8 = nullptr;
    RankParams p{};      // rank parameters of the canonical bound 8 * floor(B / 8)
    int64_t size = 0;    // |C(B)|
};

// Tables for (current device, bound), bound in [0, 40]; nullptr with err set
// on failure.  A host-side lookup: nothing is allocated or enqueued.
const DevTable* get_table(int32_t bound, e8q_status_t& err);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Blocks for a grid-stride launch of `items` work items with `per_block`
// items per block: enough to fill every CU `waves_per_cu`-deep, never more
// than there is work.
inline unsigned grid_for(uint64_t items, unsigned per_block, unsigned blocks_per_cu) {
    uint64_t need = (items + per_block - 1) / per_block;
    uint64_t cap = uint64_t(device_cu_count()) * blocks_per_cu;
    if (need < 1) need = 1;
    return unsigned(need < cap ? need : cap);
}

// Blocks of `block` threads and `lds` dynamic LDS bytes that the device keeps
// resident at once for `func` (all CUs), capped at `tiles` (at least 1).
// Kernels that loop over tiles with a grid stride are launched with exactly
// this many blocks: more would only start when resident blocks finish, i.e.
// at the end, and stretch the tail.
inline unsigned resident_grid(const void* func, unsigned block, size_t lds, uint64_t tiles) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void*, unsigned, size_t>, int> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    int per_cu = 0;
    {
        std::lock_guard<std::mutex> lk(mu);
        const auto key = std::make_tuple(dev, func, block, lds);
        auto it = cache.find(key);
        if (it != cache.end()) {
            per_cu = it->second;
        } else {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, func, int(block), lds) != hipSuccess ||
                per_cu < 1)
                per_cu = 1;
            cache.emplace(key, per_cu);
        }
    }
    const uint64_t cap = uint64_t(device_cu_count()) * uint64_t(per_cu);
    if (tiles < 1) tiles = 1;
    return unsigned(tiles < cap ? tiles : cap);
}


// First launch error of the entry point running on this thread; launch()
// records it and launch_status() reports and clears it, so a failure is
// reported by the call whose launch failed and never by a later one.
inline thread_local hipError_t g_launch_err = hipSuccess;

// Enqueues `kernel` with `args` (converted to its parameter types) and records
// a failed launch.
template <typename... KArgs, typename... Args>
inline void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st, Args&&... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<std::decay_t<KArgs>...> conv(std::forward<Args>(args)...);
    void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1] = {nullptr};
    std::apply([&argv](auto&... a) {
        size_t i = 0;
        ((argv[i++] = static_cast<void*>(&a)), ...);
    }, conv);
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, st);
    if (e != hipSuccess && g_launch_err == hipSuccess) g_launch_err = e;
}

template <typename A>
inline void launch_tiles(void (*kernel)(A), const A& args, uint64_t tiles, unsigned block, size_t lds,
                         hipStream_t st) {
    const unsigned grid = resident_grid(reinterpret_cast<const void*>(kernel), block, lds, tiles);
    launch(kernel, dim3(grid), dim3(block), lds, st, args);
}

inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Shape checks common to the projection and encode calls.  Returns E8Q_OK or
// E8Q_ERR_INVALID / E8Q_ERR_UNSUPPORTED.
inline e8q_status_t check_shape(const void* w, e8q_dtype_t w_dtype, int64_t batch, int64_t rows,
                                int64_t cols, const float* row_scale, uint32_t* status_dev) {
    if (!w || !row_scale || !status_dev) return E8Q_ERR_INVALID;
    if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 8) return E8Q_ERR_INVALID;
    if (w_dtype != E8Q_F32 && w_dtype != E8Q_BF16) return E8Q_ERR_INVALID;
    // groups of the whole call must fit 32 bits (indices are 32-bit on the device)
    const double groups = double(batch) * double(rows) * double(cols / 8);
    if (groups >= 4294967295.0) return E8Q_ERR_UNSUPPORTED;
    return E8Q_OK;
}

inline e8q_status_t check_block(const int8_t* signs, int32_t had_block, int64_t cols) {
    if (!signs) return E8Q_ERR_INVALID;
    if (!is_pow2(had_block) || had_block < 8 || had_block > 4096 || cols % had_block)
        return E8Q_ERR_INVALID;
    return E8Q_OK;
}

inline float kappa_for(int32_t had_block) {
    // fl32(1/sqrt(b)) from float64 (exact 2^-k for b = 4^k)
    return had_block > 0 ? float(1.0 / __builtin_sqrt(double(had_block))) : 1.0f;
}

// Result of the launches made since the last call (see launch()).
inline e8q_status_t launch_status() {
    const hipError_t e = g_launch_err;
    g_launch_err = hipSuccess;
    return e == hipSuccess ? E8Q_OK : E8Q_ERR_LAUNCH;
}

}  // namespace e8q
