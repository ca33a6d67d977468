// Rank tables for the finite core C(B) = { z in E8 : ||2z||^2 <= B }.
//
// E8-QAT stores each in-core group as a 16-bit index (abstract; Figure 2(c)
// caption; Table 3 checks that all core codewords decode consistently).  The
// index used here is the rank of 2z among C(B) in lexicographic order.  The
// device computes it with two table reads by splitting 2z = (tA, tB) into
// halves of four coordinates:
//
//   rank(t) = F[c][h(tA)] + G[c][ ||tA||^2 / 4 ][ (sum tA / 2) mod 2 ][ h(tB) ]
//
// c = parity class of t (all even / all odd), h() the mixed-radix index of a
// half with digits (t_i + tmax_c) / 2.  F counts core points whose first half
// is lexicographically smaller than tA; G counts admissible second halves
// smaller than tB for the state left by tA (remaining norm budget, required
// sum residue mod 4).  Both are built on the host by plain enumeration.
#pragma once

#include <stdint.h>

#include <vector>

namespace e8q {

struct RankParams {
    int32_t tm[2];       // largest |2z_i| per class (even, odd); -1 if the class is empty
    uint32_t nh[2];      // (tm+1)^4: half indices per class
    uint32_t off_f[2];   // F table offsets (entries)
    uint32_t off_g[2];   // G table offsets (entries)
    uint32_t entries;    // total uint16 entries
};

struct CoreTable {
    int32_t bound = -1;
    int64_t size = 0;            // |C(B)|
    RankParams p{};
    std::vector<uint16_t> data;  // F and G tables, laid out by RankParams
};

// Build (and self-check) the table for 0 <= bound <= 40.  Returns false if the
// self-check fails.
bool build_core_table(int32_t bound, CoreTable& out);

// Largest core bound whose table is small enough for LDS (<= 32 KB).
constexpr int32_t kLdsTableMaxBound = 31;

}  // namespace e8q
