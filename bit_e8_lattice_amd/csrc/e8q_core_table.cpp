// Host construction of the core rank tables (see e8q_core_table.hpp).
#include "e8q_core_table.hpp"

#include <array>

namespace e8q {

namespace {

using Pt = std::array<int, 8>;

// All points of C(B) in lexicographic order: coordinates are generated in
// increasing order, depth first, with the norm budget and the single-parity
// rule pruned early; the E8 sum rule (sum = 0 mod 4) is tested at the leaf.
void enumerate(int bound, int tmax, std::vector<Pt>& out) {
    Pt cur{};
    struct Rec {
        int bound, tmax;
        std::vector<Pt>* out;
        Pt* cur;
        void go(int i, int norm, int sum, int par) {
            if (i == 8) {
                if (((sum % 4) + 4) % 4 == 0) out->push_back(*cur);
                return;
            }
            for (int v = -tmax; v <= tmax; ++v) {
                if (i > 0 && ((v & 1) != par)) continue;
                const int nn = norm + v * v;
                if (nn > bound) continue;
                (*cur)[i] = v;
                go(i + 1, nn, sum + v, i == 0 ? (v & 1) : par);
            }
        }
    } r{bound, tmax, &out, &cur};
    r.go(0, 0, 0, 0);
}

uint32_t half_index(const int* t, int tm, uint32_t ub) {
    uint32_t h = 0;
    for (int i = 0; i < 4; ++i) h = h * ub + uint32_t((t[i] + tm) >> 1);
    return h;
}

}  // namespace

bool build_core_table(int32_t bound, CoreTable& out) {
    if (bound < 0 || bound > 40) return false;
    out = CoreTable{};
    out.bound = bound;
    RankParams& p = out.p;
    // even class: |t| <= largest even e with e^2 <= B; odd class: the other
    // seven coordinates are at least 1 in magnitude, so t^2 <= B - 7.
    int te = 0;
    while ((te + 2) * (te + 2) <= bound) te += 2;
    int to = -1;
    for (int o = 1; o * o + 7 <= bound; o += 2) to = o;
    p.tm[0] = te;
    p.tm[1] = to;
    p.ub = uint32_t((te > to ? te : to) + 1);
    p.nh = p.ub * p.ub * p.ub * p.ub;
    p.nstate = 2u * uint32_t(bound / 4 + 1);
    p.entries = 2u * p.nh + 2u * p.nstate * p.nh;
    out.data.assign(p.entries, uint16_t(0xFFFF));

    std::vector<Pt> pts;
    enumerate(bound, te > to ? te : to, pts);
    out.size = int64_t(pts.size());
    if (pts.size() > 0xFFFF) return false;
    out.points.assign(2 * pts.size(), 0u);
    for (size_t i = 0; i < pts.size(); ++i)
        for (int k = 0; k < 8; ++k)
            out.points[2 * i + k / 4] |= uint32_t(pts[i][k] + 64) << (8 * (k % 4));

    // F: index of the first core point with each first half.
    for (size_t i = 0; i < pts.size(); ++i) {
        const Pt& t = pts[i];
        const int c = t[0] & 1;
        uint16_t& f = out.data[uint32_t(c) * p.nh + half_index(t.data(), p.tm[c], p.ub)];
        if (f == 0xFFFF) f = uint16_t(i);
    }
    // G: running count of admissible second halves per (class, state).
    for (int c = 0; c < 2; ++c) {
        const int tm = p.tm[c];
        if (tm < 0) continue;
        for (uint32_t state = 0; state < p.nstate; ++state) {
            const int budget = bound - 2 * int(state >> 1) * 2;   // B - ||tA||^2, ||tA||^2 = 4 * (state/2)
            const int s = int(state & 1u);                         // sum tA = 2s (mod 4)
            uint32_t count = 0;
            const uint32_t row = 2u * p.nh + (uint32_t(c) * p.nstate + state) * p.nh;
            int d[4];
            for (uint32_t h = 0; h < p.nh; ++h) {
                uint32_t hh = h;
                for (int i = 3; i >= 0; --i) { d[i] = int(hh % p.ub); hh /= p.ub; }
                int norm = 0, sum = 0;
                bool ok = true;
                for (int i = 0; i < 4; ++i) {
                    if (d[i] > tm) ok = false;
                    const int t = 2 * d[i] - tm;
                    norm += t * t;
                    sum += t;
                }
                // tB must fit the remaining budget and make the total sum 0 mod 4
                if (!ok || norm > budget || (((sum + 2 * s) % 4) + 4) % 4 != 0) continue;
                out.data[row + h] = uint16_t(count);
                ++count;
            }
        }
    }
    // Self-check: the two-read formula reproduces every rank.
    for (size_t i = 0; i < pts.size(); ++i) {
        const Pt& t = pts[i];
        const int c = t[0] & 1;
        int na = 0, sa = 0;
        for (int k = 0; k < 4; ++k) { na += t[k] * t[k]; sa += t[k]; }
        const uint32_t state = uint32_t(na >> 1) + uint32_t((sa >> 1) & 1);
        const uint32_t f = out.data[uint32_t(c) * p.nh + half_index(t.data(), p.tm[c], p.ub)];
        const uint32_t g = out.data[2u * p.nh + (uint32_t(c) * p.nstate + state) * p.nh +
                                    half_index(t.data() + 4, p.tm[c], p.ub)];
        if (f + g != uint32_t(i)) return false;
    }
    return true;
}

std::vector<uint32_t> build_roots() {
    // every E8 point with ||2z||^2 = 8, enumerated in lexicographic order
    std::vector<Pt> pts;
    enumerate(8, 2, pts);
    std::vector<uint32_t> out;
    for (const Pt& t : pts) {
        int n = 0;
        for (int k = 0; k < 8; ++k) n += t[k] * t[k];
        if (n != 8) continue;
        uint32_t w[2] = {0u, 0u};
        for (int k = 0; k < 8; ++k) w[k / 4] |= uint32_t(t[k] + 64) << (8 * (k % 4));
        out.push_back(w[0]);
        out.push_back(w[1]);
    }
    return out;   // 480 words when correct
}

}  // namespace e8q
