// Table generator, run when the library is built: writes the device table
// blob (embedded by e8q_tables.hip) and a header with its layout.
//   e8q_tablegen <out_dir>  ->  <out_dir>/e8q_tables.bin, <out_dir>/e8q_tables_index.h
#include <cstdio>
#include <string>

#include "e8q_tables_build.hpp"

int main(int argc, char** argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s <out_dir>\n", argv[0]);
        return 2;
    }
    e8q::TableBlob blob;
    if (!e8q::build_table_blob(blob)) {
        std::fprintf(stderr, "e8q_tablegen: table self-check failed\n");
        return 1;
    }
    const std::string dir = argv[1];
    FILE* f = std::fopen((dir + "/e8q_tables.bin").c_str(), "wb");
    if (!f || std::fwrite(blob.bytes.data(), 1, blob.bytes.size(), f) != blob.bytes.size()) return 1;
    std::fclose(f);
    FILE* h = std::fopen((dir + "/e8q_tables_index.h").c_str(), "w");
    if (!h) return 1;
    std::fprintf(h, "// Layout of e8q_tables.bin, written by e8q_tablegen.\n#pragma once\n\n");
    std::fprintf(h, "#include \"e8q_tables_build.hpp\"\n\nnamespace e8q {\nnamespace gen {\n\n");
    std::fprintf(h, "constexpr unsigned long long kBlobBytes = %zuull;\n", blob.bytes.size());
    std::fprintf(h, "constexpr unsigned long long kRootsOffset = %lluull;\n\n",
                 (unsigned long long)blob.roots);
    std::fprintf(h, "constexpr TableSetLayout kSets[kCanonBounds] = {\n");
    for (int s = 0; s < e8q::kCanonBounds; ++s) {
        const e8q::TableSetLayout& L = blob.sets[s];
        std::fprintf(h,
                     "    {%d, %lld, {{%d, %d}, %uu, %uu, %uu, %uu}, %uu, %lluull, %lluull, %lluull, %lluull, "
                     "%lluull, %lluull},\n",
                     L.bound, (long long)L.size, L.p.tm[0], L.p.tm[1], L.p.ub, L.p.nh, L.p.nstate, L.p.entries,
                     L.ntiles, (unsigned long long)L.rank, (unsigned long long)L.points,
                     (unsigned long long)L.h8, (unsigned long long)L.pbf, (unsigned long long)L.p64,
                     (unsigned long long)L.tiles);
    }
    std::fprintf(h, "};\n\n}  // namespace gen\n}  // namespace e8q\n");
    std::fclose(h);
    return 0;
}
