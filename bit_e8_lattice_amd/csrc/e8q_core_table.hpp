// Rank tables for the finite core C(B) = { z in E8 : ||2z||^2 <= B }.
//
// E8-QAT stores each in-core group as a 16-bit index (abstract; Figure 2(c)
// caption; Table 3 checks that all core codewords decode consistently).  The
// index used here is the rank of t = 2z among C(B) in lexicographic order.
// The device computes it with two table reads by splitting t = (tA, tB) into
// halves of four coordinates:
//
//   rank(t) = F[c][h(tA)] + G[c][state(tA)][h(tB)]
//
// c = parity class of t (0: all even, 1: all odd).  Digits d_i = (t_i +
// tm_c) / 2 lie in [0, tm_c], where tm_c is the largest |t_i| a core point of
// class c can have; both classes use one radix ub = max(tm_0, tm_1) + 1, so
// h(.) = sum d_i ub^(3-i) < ub^4 = nh.  F counts core points whose first
// half is lexicographically smaller than tA.  state = ||tA||^2 / 2 +
// ((sum tA / 2) mod 2) encodes what tA leaves for tB (norm budget, required
// sum residue mod 4); G counts admissible second halves smaller than tB.
//
// Layout (uint16 entries): F[c] at c*nh, G[c][state] at 2*nh + (c*nstate +
// state)*nh, nstate = 2*(B/4 + 1).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace e8q {

struct RankParams {
    int32_t tm[2];       // largest |t_i| per class (even, odd); -1 if the class is empty
    uint32_t ub;         // digit radix shared by both classes
    uint32_t nh;         // ub^4
    uint32_t nstate;     // 2 * (bound/4 + 1)
    uint32_t entries;    // 2*nh + 2*nstate*nh
};

struct CoreTable {
    int32_t bound = -1;
    int64_t size = 0;            // |C(B)|
    RankParams p{};
    std::vector<uint16_t> data;
    // Points in rank order, two words each: bytes 2z_i + 64, coordinates 0-3
    // in the first word and 4-7 in the second (low byte first).
    std::vector<uint32_t> points;
};

// Build (and self-check) the table for 0 <= bound <= 40.  Returns false if the
// self-check fails.
bool build_core_table(int32_t bound, CoreTable& out);

// The 240 roots of E8 (||r||^2 = 2) as 2r, in lexicographic order (signed,
// coordinate 0 most significant), two words each with bytes 2r_i + 64 as in
// CoreTable::points.
std::vector<uint32_t> build_roots();

}  // namespace e8q
