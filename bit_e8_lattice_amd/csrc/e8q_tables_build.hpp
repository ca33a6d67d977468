// Build-time construction of every read-only device table the library uses.
//
// The tables depend only on the core bound, and only through the core set
// C(B) = { z in E8 : ||2z||^2 <= B }.  ||2z||^2 = 4 ||z||^2 is a multiple of 8
// for every E8 point (||z||^2 is even), so C(B) = C(8 * floor(B / 8)) and six
// table sets (B = 0, 8, 16, 24, 32, 40) serve every bound the library accepts.
// The generator program (e8q_tablegen.cpp) runs these builders when the
// library is compiled and writes one binary blob, which e8q_tables.hip embeds
// in the device code object, plus a header of offsets and rank parameters.
// No call of the library ever allocates, uploads or synchronizes for a table.
#pragma once

#include <stdint.h>

#include <vector>

#include "e8q_core_table.hpp"

namespace e8q {

constexpr uint32_t kTileRows = 32;    // core points per tile of the PTQ's matrix-core search
constexpr int kCanonBounds = 6;       // canonical bounds 0, 8, ..., 40

// Where one canonical bound's tables sit in the blob (byte offsets, each
// 256-byte aligned), with its rank parameters.
struct TableSetLayout {
    int32_t bound;
    int64_t size;        // |C(B)|
    RankParams p;
    uint32_t ntiles;     // PTQ search tiles
    uint64_t rank;       // uint16 [p.entries]: the two-read rank table
    uint64_t points;     // uint32 [2 * size]: 2z + 64 as bytes, coordinates 0-3 then 4-7
    uint64_t h8;         // uint32 [2 * size]: H_8 (2z) as signed bytes, same word layout
    uint64_t pbf;        // uint16 [8 * (size + 1)]: 2z as bfloat16, plus a zero entry at index size
    uint64_t p64;        // double [9 * size]: 2z as doubles, then ||2z||^2 / 4
    uint64_t tiles;      // uint8 [900 * ntiles]: PTQ shell tiles (layout in e8q_host.hpp)
};

struct TableBlob {
    std::vector<uint8_t> bytes;
    TableSetLayout sets[kCanonBounds];
    uint64_t roots;      // uint32 [480]: the 240 roots as 2r + 64 bytes, lexicographic order
};

// Builds (and self-checks) every table.  Returns false if a self-check fails.
bool build_table_blob(TableBlob& out);

}  // namespace e8q
