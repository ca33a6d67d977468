// Host-only entry points and shared host state.
#include <atomic>
#include <cstddef>
#include <cstring>
#include <map>
#include <unordered_map>
#include <mutex>

#include "e8q_core_table.hpp"
#include "e8q_host.hpp"

// The record layouts are part of the ABI (kernels read and write them as
// 32-bit words).
static_assert(sizeof(e8q_escape_t) == 20 && alignof(e8q_escape_t) == 4, "escape record layout");
static_assert(offsetof(e8q_escape_t, two_z) == 4, "escape record layout");
static_assert(sizeof(e8q_escape_packed_t) == 8, "packed record layout");
static_assert(offsetof(e8q_escape_packed_t, core_idx) == 4 && offsetof(e8q_escape_packed_t, root) == 6,
              "packed record layout");

namespace e8q {

int64_t core_size_host(int32_t bound);

namespace {
std::mutex g_tab_mu;
std::map<std::pair<int, int>, DevTable>* g_tabs = nullptr;

template <typename T>
bool upload(const std::vector<T>& v, T*& dptr) {
    const size_t bytes = v.size() * sizeof(T);
    if (hipMalloc(&dptr, bytes) != hipSuccess) return false;
    if (hipMemcpy(dptr, v.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(dptr);
        dptr = nullptr;
        return false;
    }
    return true;
}
// The tile tables of DevTable: shells ||t||^2 = 0, 8, 16, ... in increasing
// norm; of each pair +-t only t with its first nonzero coordinate positive
// (the origin alone in its shell), in rank order, cut into tiles of kTileRows
// rows (pads after the shell's last point); each row also names the core
// index of -t.
std::vector<uint8_t> build_tiles(const CoreTable& c, uint32_t& ntiles) {
    auto coord = [&](int64_t i, int k) { return int((c.points[2 * i + k / 4] >> (8 * (k % 4))) & 0xFFu) - 64; };
    auto key = [](const int (&t)[8]) {
        uint64_t k = 0;
        for (int i = 0; i < 8; ++i) k = (k << 8) | uint64_t(uint8_t(t[i] + 64));
        return k;
    };
    std::unordered_map<uint64_t, int64_t> where;
    std::vector<std::vector<int64_t>> shells(size_t(c.bound / 8) + 1);
    int64_t origin = -1;
    for (int64_t i = 0; i < c.size; ++i) {
        int t[8], n = 0, first = 0;
        for (int k = 0; k < 8; ++k) {
            t[k] = coord(i, k);
            n += t[k] * t[k];
            if (first == 0) first = t[k];
        }
        where[key(t)] = i;
        if (n == 0) origin = i;
        if (first >= 0) shells[size_t(n / 8)].push_back(i);   // the origin, or t with first nonzero > 0
    }
    std::vector<int64_t> rows;    // -1 = pad
    std::vector<float> n4;
    for (size_t s = 0; s < shells.size(); ++s) {
        const auto& sh = shells[s];
        if (sh.empty()) continue;
        const size_t nt = (sh.size() + kTileRows - 1) / kTileRows;
        for (size_t j = 0; j < nt * kTileRows; ++j) rows.push_back(j < sh.size() ? sh[j] : -1);
        for (size_t j = 0; j < nt; ++j) n4.push_back(float(s * 8) / 4.0f);
    }
    // an even tile count (the search takes two tiles per step): a dummy tile
    // of pads whose key can never be the best
    if (n4.size() % 2) {
        for (size_t j = 0; j < kTileRows; ++j) rows.push_back(-1);
        n4.push_back(1e30f);
    }
    ntiles = uint32_t(n4.size());
    const size_t nt = ntiles;
    std::vector<uint8_t> out(nt * 900, 0);
    uint16_t* bf = reinterpret_cast<uint16_t*>(out.data());
    int8_t* t8 = reinterpret_cast<int8_t*>(out.data() + nt * 512);
    uint16_t* ipos = reinterpret_cast<uint16_t*>(out.data() + nt * 768);
    uint16_t* ineg = reinterpret_cast<uint16_t*>(out.data() + nt * 832);
    float* nf = reinterpret_cast<float*>(out.data() + nt * 896);
    for (size_t r = 0; r < rows.size(); ++r) {
        const int64_t i = rows[r];
        int t[8], m[8];
        for (int k = 0; k < 8; ++k) {
            t[k] = i < 0 ? 0 : coord(i, k);
            m[k] = -t[k];
        }
        ipos[r] = uint16_t(i < 0 ? origin : i);
        ineg[r] = uint16_t(i < 0 ? origin : where.at(key(m)));
        for (int k = 0; k < 8; ++k) {
            const float f = float(t[k]);
            uint32_t u;
            std::memcpy(&u, &f, 4);
            bf[r * 8 + k] = uint16_t(u >> 16);   // small integers are exact in bf16
            t8[r * 8 + k] = int8_t(t[k]);
        }
    }
    std::memcpy(nf, n4.data(), nt * 4);
    return out;
}
}  // namespace

const DevTable* get_table(int32_t bound, e8q_status_t& err) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        err = E8Q_ERR_DEVICE;
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_tab_mu);
    if (!g_tabs) g_tabs = new std::map<std::pair<int, int>, DevTable>();
    auto key = std::make_pair(dev, int(bound));
    auto it = g_tabs->find(key);
    if (it != g_tabs->end()) return &it->second;
    DevTable t;
    if (!build_core_table(bound, t.host) || !upload(t.host.data, t.dptr)) {
        err = E8Q_ERR_DEVICE;
        return nullptr;
    }
    const std::vector<uint32_t> roots = build_roots();
    if (roots.size() != 480 || !upload(t.host.points, t.dpoints)) {
        (void)hipFree(t.dptr);
        err = E8Q_ERR_DEVICE;
        return nullptr;
    }
    std::vector<double> p64(size_t(t.host.size) * 9, 0.0);
    for (int64_t i = 0; i < t.host.size; ++i) {
        double n = 0.0;
        for (int k = 0; k < 8; ++k) {
            const int v = int((t.host.points[2 * i + k / 4] >> (8 * (k % 4))) & 0xFFu) - 64;
            p64[size_t(i) * 9 + k] = double(v);
            n += double(v * v);
        }
        p64[size_t(i) * 9 + 8] = n / 4.0;
    }
    std::vector<uint8_t> tiles = build_tiles(t.host, t.ntiles);
    std::vector<uint16_t> pbf((size_t(t.host.size) + 1) * 8, 0);
    for (size_t i = 0; i < size_t(t.host.size) * 8; ++i) {
        const float f = float(p64[(i / 8) * 9 + i % 8]);
        uint32_t u;
        std::memcpy(&u, &f, 4);
        pbf[i] = uint16_t(u >> 16);   // small integers are exact in bf16
    }
    std::vector<uint32_t> h8(size_t(t.host.size) * 2, 0u);
    for (int64_t i = 0; i < t.host.size; ++i) {
        int v[8];
        for (int k = 0; k < 8; ++k) v[k] = int(p64[size_t(i) * 9 + k]);
        for (int h = 1; h < 8; h <<= 1)
            for (int k = 0; k < 8; ++k)
                if ((k & h) == 0) {
                    const int a = v[k], b = v[k + h];
                    v[k] = a + b;
                    v[k + h] = a - b;
                }
        for (int k = 0; k < 8; ++k) h8[size_t(i) * 2 + k / 4] |= (uint32_t(v[k]) & 0xFFu) << (8 * (k % 4));
    }
    uint16_t* dpbf = nullptr;
    if (!upload(roots, t.droots) || !upload(p64, t.dpts64) || !upload(tiles, t.dtiles) || !upload(pbf, dpbf) ||
        !upload(h8, t.dh8)) {
        (void)hipFree(t.dptr);
        (void)hipFree(t.dpoints);
        if (t.droots) (void)hipFree(t.droots);
        if (t.dpts64) (void)hipFree(t.dpts64);
        if (t.dtiles) (void)hipFree(t.dtiles);
        if (dpbf) (void)hipFree(dpbf);
        err = E8Q_ERR_DEVICE;
        return nullptr;
    }
    t.dpts_bf16 = reinterpret_cast<uint4*>(dpbf);
    auto res = g_tabs->emplace(key, std::move(t));
    return &res.first->second;
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
