// Build-time construction of the device tables (see e8q_tables_build.hpp).
#include "e8q_tables_build.hpp"

#include <cstring>
#include <unordered_map>

namespace e8q {

namespace {

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

template <typename T>
uint64_t append(std::vector<uint8_t>& blob, const std::vector<T>& v) {
    const uint64_t off = (blob.size() + 255) & ~uint64_t(255);
    blob.resize(off + v.size() * sizeof(T), 0);
    std::memcpy(blob.data() + off, v.data(), v.size() * sizeof(T));
    return off;
}

}  // namespace

bool build_table_blob(TableBlob& out) {
    out.bytes.clear();
    for (int s = 0; s < kCanonBounds; ++s) {
        CoreTable c;
        if (!build_core_table(8 * s, c)) return false;
        TableSetLayout& L = out.sets[s];
        L.bound = c.bound;
        L.size = c.size;
        L.p = c.p;
        // the points as doubles (2z, then ||2z||^2 / 4), as bfloat16 (plus a
        // zero entry), and their natural-order 8-point Walsh-Hadamard
        // transforms (exact small integers) as signed bytes
        std::vector<double> p64(size_t(c.size) * 9, 0.0);
        std::vector<uint16_t> pbf((size_t(c.size) + 1) * 8, 0);
        std::vector<uint32_t> h8(size_t(c.size) * 2, 0u);
        for (int64_t i = 0; i < c.size; ++i) {
            int v[8];
            double n = 0.0;
            for (int k = 0; k < 8; ++k) {
                v[k] = int((c.points[2 * i + k / 4] >> (8 * (k % 4))) & 0xFFu) - 64;
                p64[size_t(i) * 9 + k] = double(v[k]);
                n += double(v[k] * v[k]);
                const float f = float(v[k]);
                uint32_t u;
                std::memcpy(&u, &f, 4);
                pbf[size_t(i) * 8 + k] = uint16_t(u >> 16);   // small integers are exact in bf16
            }
            p64[size_t(i) * 9 + 8] = n / 4.0;
            for (int h = 1; h < 8; h <<= 1)
                for (int k = 0; k < 8; ++k)
                    if ((k & h) == 0) {
                        const int a = v[k], b = v[k + h];
                        v[k] = a + b;
                        v[k + h] = a - b;
                    }
            for (int k = 0; k < 8; ++k) h8[size_t(i) * 2 + k / 4] |= (uint32_t(v[k]) & 0xFFu) << (8 * (k % 4));
        }
        const std::vector<uint8_t> tiles = build_tiles(c, L.ntiles);
        L.rank = append(out.bytes, c.data);
        L.points = append(out.bytes, c.points);
        L.h8 = append(out.bytes, h8);
        L.pbf = append(out.bytes, pbf);
        L.p64 = append(out.bytes, p64);
        L.tiles = append(out.bytes, tiles);
    }
    const std::vector<uint32_t> roots = build_roots();
    if (roots.size() != 480) return false;
    out.roots = append(out.bytes, roots);
    out.bytes.resize((out.bytes.size() + 255) & ~size_t(255), 0);
    return true;
}

}  // namespace e8q
