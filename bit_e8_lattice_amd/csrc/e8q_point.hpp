// Per-group pipeline shared by the projection and encode kernels: load,
// randomized Walsh-Hadamard rotation (any block 8..4096), and the nearest E8
// point on a fast packed path or the exact path.
//
// Both kernels run 512-thread blocks over tiles of 4096 consecutive groups:
// item j of a tile is the 512 groups tile*4096 + j*512 + [0, 512); inside an
// item, thread (wave w, lane l) owns group w*64 + (l & ~15) + logical(l).
// Blocks up to 128 columns are rotated in registers (in-lane + DPP stages);
// wider blocks finish their stages after an LDS transpose, which needs every
// thread of the block to call the rotation together.
#pragma once

#include "e8q_core_table.hpp"
#include "e8q_device.hpp"

namespace e8q {

constexpr int kBlock = 512;
constexpr int kWaves = kBlock / kWave;
constexpr int kItems = 8;                          // groups per thread per tile
constexpr uint32_t kTileGroups = kItems * kBlock;  // 4096
constexpr float kMagic = 12582944.0f;              // 1.5 * 2^23 + 32
constexpr float kFastXMax = 30.0f;

// Raw input of one group: 16 bytes of bf16 (or 32 bytes of float32).
struct Raw {
    uint4 p;
    uint4 q;   // second half, float32 input only
};

template <typename WT>
__device__ __forceinline__ Raw load_raw(const void* w, uint32_t g) {
    Raw r;
    if constexpr (sizeof(WT) == 2) {
        r.p = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(w) + uint64_t(g) * 8);
        r.q = make_uint4(0u, 0u, 0u, 0u);
    } else {
        const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(w) + uint64_t(g) * 8);
        r.p = src[0];
        r.q = src[1];
    }
    return r;
}

// Remaining butterfly stages of 256- and 512-column blocks, inside the wave:
// stride 128 pairs lane l with lane l ^ 16 (the same logical position in the
// next 16-lane row), stride 256 lane l with l ^ 32.  v holds the true values
// (lane sign already removed); every lane of the wave takes part.  The lower
// lane keeps p + q, the upper one p - q (one rounding each, as a butterfly).
template <int HB>
__device__ __forceinline__ void wave_stages(float (&v)[8]) {
    const uint32_t lane = __lane_id();
#pragma unroll
    for (int m = 16; m < HB / 8; m <<= 1) {
        const float eps = (lane & uint32_t(m)) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float o = __shfl_xor(v[i], m, 64);
            v[i] = fmaf(eps, v[i], o);
        }
    }
}

// Remaining butterfly stages of blocks wider than 128 columns: stride
// 128 * 2^k for k = 0 .. log2(HB/128) - 1, in that order.  v holds the true
// values (lane sign already removed) of this thread's group; lpos is the
// group's position inside the item.  s_wide: 8 * kBlock floats of LDS.
template <int HB, int S = 128>
__device__ __forceinline__ void wide_stages(float (&v)[8], float* s_wide, uint32_t lpos, uint32_t tid) {
    constexpr int M = HB / S;            // S-column sub-blocks per block (stages of stride S, 2S, ...)
    constexpr int TPB = HB / 8;          // threads per block
#pragma unroll
    for (int i = 0; i < 8; ++i) s_wide[lpos * 8 + i] = v[i];
    __syncthreads();
    const uint32_t bi = tid / TPB, r = tid % TPB;
    float* blk = s_wide + bi * HB;
    float u[8];
    if constexpr (M <= 8) {
        // 8/M positions per thread (r, r + TPB, ...: neighbouring threads read
        // neighbouring words), all M sub-blocks of each
        constexpr int P = 8 / M;
#pragma unroll
        for (int pp = 0; pp < P; ++pp)
#pragma unroll
            for (int s = 0; s < M; ++s) u[pp * M + s] = blk[s * S + pp * TPB + r];
#pragma unroll
        for (int h = 1; h < M; h <<= 1)
#pragma unroll
            for (int pp = 0; pp < P; ++pp)
#pragma unroll
                for (int s = 0; s < M; ++s)
                    if ((s & h) == 0) {
                        const float p = u[pp * M + s], q = u[pp * M + s + h];
                        u[pp * M + s] = p + q;
                        u[pp * M + s + h] = p - q;
                    }
        __syncthreads();
#pragma unroll
        for (int pp = 0; pp < P; ++pp)
#pragma unroll
            for (int s = 0; s < M; ++s) blk[s * S + pp * TPB + r] = u[pp * M + s];
    } else {
        static_assert(S == 128, "sub-blocks of S columns with S > 128 number at most 8");
        // one position, sub-blocks qt*8 .. qt*8+7 in-thread, qt across M/8 adjacent lanes
        constexpr int T = M / 8;
        const uint32_t pos = r / T, qt = r % T;
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = blk[(qt * 8 + i) * 128 + pos];
#pragma unroll
        for (int h = 1; h < 8; h <<= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((i & h) == 0) {
                    const float p = u[i], q = u[i + h];
                    u[i] = p + q;
                    u[i + h] = p - q;
                }
#pragma unroll
        for (int m = 1; m < T; m <<= 1) {
            const bool low = (qt & m) == 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float o = __shfl_xor(u[i], m, 64);
                u[i] = low ? (u[i] + o) : (o - u[i]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) blk[(qt * 8 + i) * 128 + pos] = u[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s_wide[lpos * 8 + i];
    __syncthreads();   // the buffer is reused by the next item
}

// Butterfly stages of stride >= 8 (across lanes, then through LDS for blocks
// wider than 128 columns) on values whose in-lane stages are done.  Returns
// the sign bit that the lane's results carry (see fwht_xlane).  Same calling
// rules as rotate_group.
template <int HB>
__device__ __forceinline__ uint32_t fwht_cross(float (&v)[8], const LaneFwht& lf, float* s_wide, uint32_t lpos,
                                               uint32_t tid) {
    constexpr int RB = HB > 128 ? 128 : HB;
    fwht_xlane<RB>(v, lf.eps);
    if constexpr (HB > 128) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(__float_as_uint(v[i]) ^ lf.sign);
        // 256 and 512 columns: inside the wave.  4096: strides 128 and 256
        // inside the wave, the rest through LDS over 512-column sub-blocks (one
        // position per thread).  1024 and 2048: all through LDS (measured
        // faster than with the shuffles first).
        if constexpr (HB <= 512) {
            wave_stages<HB>(v);
        } else if constexpr (HB >= 4096) {
            wave_stages<512>(v);
            wide_stages<HB, 512>(v, s_wide, lpos, tid);
        } else {
            wide_stages<HB>(v, s_wide, lpos, tid);
        }
        return 0u;
    } else {
        return HB >= 16 ? lf.sign : 0u;
    }
}

// Whole Walsh-Hadamard transform of the block holding this thread's group.
template <int HB>
__device__ __forceinline__ uint32_t fwht_group(float (&v)[8], const LaneFwht& lf, float* s_wide, uint32_t lpos,
                                               uint32_t tid) {
    fwht_inlane<(HB > 128 ? 128 : HB)>(v);
    return fwht_cross<HB>(v, lf, s_wide, lpos, tid);
}

// Widen one group's raw input to float32 (no sign flip).
template <typename WT>
__device__ __forceinline__ void widen_raw(const Raw& r, float (&v)[8]) {
    if constexpr (sizeof(WT) == 2) {
        v[0] = __uint_as_float(r.p.x << 16); v[1] = __uint_as_float(r.p.x & 0xFFFF0000u);
        v[2] = __uint_as_float(r.p.y << 16); v[3] = __uint_as_float(r.p.y & 0xFFFF0000u);
        v[4] = __uint_as_float(r.p.z << 16); v[5] = __uint_as_float(r.p.z & 0xFFFF0000u);
        v[6] = __uint_as_float(r.p.w << 16); v[7] = __uint_as_float(r.p.w & 0xFFFF0000u);
    } else {
        v[0] = __uint_as_float(r.p.x); v[1] = __uint_as_float(r.p.y);
        v[2] = __uint_as_float(r.p.z); v[3] = __uint_as_float(r.p.w);
        v[4] = __uint_as_float(r.q.x); v[5] = __uint_as_float(r.q.y);
        v[6] = __uint_as_float(r.q.z); v[7] = __uint_as_float(r.q.w);
    }
}

// Flip the float32 sign bits of one group by its column signs (mask words as
// stored in LDS: bit 15 / bit 31 of word k for columns 2k / 2k+1).
__device__ __forceinline__ void flip_f32(float (&y)[8], const uint4& m) {
    y[0] = __uint_as_float(__float_as_uint(y[0]) ^ (m.x << 16)); y[1] = __uint_as_float(__float_as_uint(y[1]) ^ (m.x & 0x80000000u));
    y[2] = __uint_as_float(__float_as_uint(y[2]) ^ (m.y << 16)); y[3] = __uint_as_float(__float_as_uint(y[3]) ^ (m.y & 0x80000000u));
    y[4] = __uint_as_float(__float_as_uint(y[4]) ^ (m.z << 16)); y[5] = __uint_as_float(__float_as_uint(y[5]) ^ (m.z & 0x80000000u));
    y[6] = __uint_as_float(__float_as_uint(y[6]) ^ (m.w << 16)); y[7] = __uint_as_float(__float_as_uint(y[7]) ^ (m.w & 0x80000000u));
}

// Column-sign mask words of LDS for `cols` columns (signs: +-1 int8).
__device__ __forceinline__ void load_sign_masks(uint32_t* s_smask, const int8_t* signs, uint32_t cols, uint32_t tid) {
    for (uint32_t i = tid; i < cols / 2u; i += kBlock) {
        const uint32_t s0 = uint32_t(uint8_t(signs[2 * i])) >> 7;
        const uint32_t s1 = uint32_t(uint8_t(signs[2 * i + 1])) >> 7;
        s_smask[i] = (s0 << 15) | (s1 << 31);
    }
}

// Sign flip, widen and Walsh-Hadamard rotation of one group.  Returns in v
// the rotated values times (-1)^vsign-bit: multiply by the coefficient with
// that sign bit applied.  All threads of the block must call this together
// (wide blocks) and all lanes of each wave must be active (DPP stages).
template <typename WT, int HB>
__device__ __forceinline__ uint32_t rotate_group(const uint32_t* s_smask, float* s_wide, Raw r, uint32_t col_group,
                                                 const LaneFwht& lf, uint32_t lpos, uint32_t tid, float (&v)[8]) {
    if constexpr (HB > 0) {
        const uint4 m = *reinterpret_cast<const uint4*>(s_smask + col_group * 4u);
        if constexpr (sizeof(WT) == 2) {
            r.p.x ^= m.x; r.p.y ^= m.y; r.p.z ^= m.z; r.p.w ^= m.w;
        } else {
            r.p.x ^= m.x << 16; r.p.y ^= m.x & 0x80000000u;
            r.p.z ^= m.y << 16; r.p.w ^= m.y & 0x80000000u;
            r.q.x ^= m.z << 16; r.q.y ^= m.z & 0x80000000u;
            r.q.z ^= m.w << 16; r.q.w ^= m.w & 0x80000000u;
        }
    }
    widen_raw<WT>(r, v);
    return fwht_group<HB>(v, lf, s_wide, lpos, tid);
}

// Exact lattice point from normalized coordinates (invalid data -> 0).
__device__ __forceinline__ uint32_t exact_point(const float (&x)[8], bool bad_row, int (&t)[8]) {
    const uint32_t inv = bad_row ? uint32_t(E8Q_STATUS_BAD_SCALE) : group_invalid_bits(x);
    if (inv) {
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = 0;
    } else {
        nearest_e8(x, t);
    }
    return inv;
}

__device__ __forceinline__ uint32_t norm_u32(const int (&t)[8]) {
    uint32_t n = 0;   // <= 8 * 16386^2 < 2^32
#pragma unroll
    for (int i = 0; i < 8; ++i) n += uint32_t(t[i] * t[i]);
    return n;
}

// Rank of a core point (|t_i| <= tm of its class) in the unified table layout.
__device__ __forceinline__ uint32_t core_rank(const int (&t)[8], const uint16_t* tab, const RankParams& p) {
    const uint32_t c = uint32_t(t[0]) & 1u;
    const int tm = c ? p.tm[1] : p.tm[0];
    uint32_t ha = 0, hb = 0;
    int na = 0, sa = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ha = ha * p.ub + uint32_t((t[i] + tm) >> 1);
        hb = hb * p.ub + uint32_t((t[4 + i] + tm) >> 1);
        na += t[i] * t[i];
        sa += t[i];
    }
    const uint32_t state = uint32_t(na >> 1) + (uint32_t(sa >> 1) & 1u);
    return uint32_t(tab[c * p.nh + ha]) + uint32_t(tab[2u * p.nh + (c * p.nstate + state) * p.nh + hb]);
}

// Fast path for one group (see the encode kernel's header for the method).
// Returns false when the group must take the exact path.  On success t0/t1
// hold 2z + 64 as bytes (coordinates 0-3 in t0, 4-7 in t1) and d8 tells the
// coset (D8 when true).
__device__ __forceinline__ bool fast_point(const float (&x)[8], uint32_t& t0, uint32_t& t1, bool& d8) {
    float d[8];
    uint32_t yb[8], db[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float y = x[i] + kMagic;     // low byte of the bits: rint(x) + 32
        d[i] = x[i] - (y - kMagic);
        yb[i] = __float_as_uint(y);
        db[i] = __float_as_uint(d[i]);
    }
    // n_i + 32 bytes and (d_i < 0 ? 0xFF : 0) bytes, four per word
    const uint32_t n0 = __builtin_amdgcn_perm(yb[1], yb[0], 0x0C0C0400u) | __builtin_amdgcn_perm(yb[3], yb[2], 0x04000C0Cu);
    const uint32_t n1 = __builtin_amdgcn_perm(yb[5], yb[4], 0x0C0C0400u) | __builtin_amdgcn_perm(yb[7], yb[6], 0x04000C0Cu);
    const uint32_t m0 = __builtin_amdgcn_perm(db[1], db[0], 0x0C0C0B09u) | __builtin_amdgcn_perm(db[3], db[2], 0x0B090C0Cu);
    const uint32_t m1 = __builtin_amdgcn_perm(db[5], db[4], 0x0C0C0B09u) | __builtin_amdgcn_perm(db[7], db[6], 0x0B090C0Cu);
    // parity of sum(n) and of sum(floor) = sum(n) - #(d < 0): byte sums with
    // v_sad_u8 (sum of |byte - 0|; it pairs with other VALU instructions,
    // v_dot4 does not), where a 0xFF byte of m adds 255, as odd as 1
    const uint32_t nsum = __builtin_amdgcn_sad_u8(n0, 0u, __builtin_amdgcn_sad_u8(n1, 0u, 0u));
    const uint32_t fsum = __builtin_amdgcn_sad_u8(m0, 0u, __builtin_amdgcn_sad_u8(m1, 0u, nsum));
    const bool odd0 = (nsum & 1u) != 0u;
    const bool odd1 = (fsum & 1u) != 0u;
    const float sa = ((fabsf(d[0]) + fabsf(d[1])) + (fabsf(d[2]) + fabsf(d[3]))) +
                     ((fabsf(d[4]) + fabsf(d[5])) + (fabsf(d[6]) + fabsf(d[7])));
    const float amax = fmaxf(fmaxf(fmaxf(fabsf(d[0]), fabsf(d[1])), fmaxf(fabsf(d[2]), fabsf(d[3]))),
                             fmaxf(fmaxf(fabsf(d[4]), fabsf(d[5])), fmaxf(fabsf(d[6]), fabsf(d[7]))));
    const float amin = fminf(fminf(fminf(fabsf(d[0]), fabsf(d[1])), fminf(fabsf(d[2]), fabsf(d[3]))),
                             fminf(fminf(fabsf(d[4]), fabsf(d[5])), fminf(fabsf(d[6]), fabsf(d[7]))));
    const float xmax = fmaxf(fmaxf(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fabsf(x[2])),
                                   fmaxf(fmaxf(fabsf(x[3]), fabsf(x[4])), fabsf(x[5]))),
                             fmaxf(fabsf(x[6]), fabsf(x[7])));
    // coset decision in float32 (trusted when clear of its rounding error)
    const float tq0 = sa - 2.0f;
    const float tq1 = odd0 ? tq0 + fmaf(-2.0f, amax, 1.0f) : tq0;
    const float tq = odd1 ? fmaf(-2.0f, amin, tq1) : tq1;
    const bool fast = (xmax < kFastXMax) && (amin > 0.0f) && (fabsf(tq) > kFastDecision);
    d8 = tq < 0.0f;
    const bool fixon = (d8 && odd0) || (!d8 && odd1);   // lane masks: scalar logic
    if (!fast) return false;
    // e_i = w |d_i| + u is +0 exactly where |d_i| equals the target (the
    // largest |d| for D8, the smallest for D8+1/2) and negative elsewhere (one
    // rounding of an exact difference keeps its sign); -inf everywhere when
    // the candidate's parity needs no fix
    const float w = d8 ? 1.0f : -1.0f;
    const float u = fixon ? (d8 ? -amax : amin) : -__builtin_inff();
    uint32_t eb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) eb[i] = __float_as_uint(fmaf(fabsf(d[i]), w, u));
    // 0xFF bytes where e_i < 0, then 0x01 at the first (lowest-index) byte
    // that is 0x00, if any: ~ne & (ne + 1) over the 64-bit pair
    const uint32_t ne0 = __builtin_amdgcn_perm(eb[1], eb[0], 0x0C0C0B09u) | __builtin_amdgcn_perm(eb[3], eb[2], 0x0B090C0Cu);
    const uint32_t ne1 = __builtin_amdgcn_perm(eb[5], eb[4], 0x0C0C0B09u) | __builtin_amdgcn_perm(eb[7], eb[6], 0x0B090C0Cu);
    const uint64_t ne = (uint64_t(ne1) << 32) | ne0;
    const uint64_t lb = ~ne & (ne + 1ull);
    const uint32_t l0 = uint32_t(lb), l1 = uint32_t(lb >> 32);
    // 2z + 64: D8 -> 2(n + 32); D8+1/2 -> 2(n + 32) + 1 - 2[d < 0].  The fix
    // moves the coordinate by +2 sgn(d) (D8) or -2 sgn(d) (D8+1/2): by -2
    // where X = m ^ (D8 ? 0 : ~0) has 0xFF, else by +2, i.e. + 2 l - 4 (l & X).
    // Every byte stays in [2, 126] (|n| <= 30), so no carry or borrow crosses
    // a byte.
    const uint32_t dm = d8 ? 0u : 0xFFFFFFFFu;
    const uint32_t hb = dm & 0x01010101u, hn = dm & 0x02020202u;
    t0 = (((n0 << 1) | hb) + (l0 << 1)) - ((m0 & hn) + ((l0 & (m0 ^ dm)) << 2));
    t1 = (((n1 << 1) | hb) + (l1 << 1)) - ((m1 & hn) + ((l1 & (m1 ^ dm)) << 2));
    return true;
}

}  // namespace e8q
