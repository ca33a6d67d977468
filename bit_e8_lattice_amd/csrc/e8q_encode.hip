// e8q_encode_core_escape: export encoding into 16-bit core indices plus
// compacted exact escape records.
//
// E8-QAT keeps the final lattice points exactly: a 2-bit-per-weight core index
// per group and a sparse 20-byte record for each group outside the finite
// core (abstract; Figure 2(c) and Figure 6(c) captions; Table 10).
//
// One pass over the weights.  Blocks claim tiles of consecutive groups in
// increasing order from a device-wide counter.  Pass 1 over a tile computes
// every lattice point and core index, stores the indices and counts escapes
// (wave ballots); a block scan plus a decoupled look-back over per-tile status
// words (aggregate / inclusive prefix, packed with their flag in one 64-bit
// word) gives the tile's first record slot.  Pass 1 also lists the tile's
// first kStagedRecs escapes (group, 2z) in LDS; a tile with no more escapes
// than that writes its records from the list, ranked by group.  Otherwise
// pass 2 recomputes only the (item, wave) slices that contain escapes -- their
// weights are still in L2 -- and writes the records.  Record order is
// therefore ascending group order whatever the scheduling.  Only tiles with more than kStagedRecs escapes,
// and every kAnchorTiles-th tile, resolve their prefix there; every other
// tile publishes its aggregate and goes on without waiting for its
// predecessors, staging its (at most kStagedRecs) records in the workspace.
// A second kernel then places the staged records: the anchors' inclusive
// prefixes plus a scan of the per-tile counts give every tile's first slot.
//
// The lattice point of a group is computed on one of two paths that give the
// same result:
//  * fast path (bf16 input, core bound <= 31, every |x_i| < 30, no x_i an
//    integer, coset decision clear of float32 rounding): rint by the magic
//    constant 1.5*2^23 + 32, whose low byte is then n_i + 32; the candidates
//    2z + 64 are assembled four coordinates per 32-bit word with v_perm, the
//    parity fix is located with per-element lane masks (first match = lowest
//    index) and applied as a +-2 byte delta; squares and the two table
//    indices come from v_dot4_u32_u8 on the packed words, byte sums from
//    v_sad_u8;
//  * exact path (everything else, and the escape records): the decoder of
//    nearest_e8() on eight int32 coordinates, float64 decision when close.
#include <map>
#include <mutex>
#include <utility>

#include "e8q_core_table.hpp"
#include "e8q_device.hpp"
#include "e8q_host.hpp"
#include "e8q_point.hpp"

namespace e8q {

constexpr uint64_t kFlagA = 1ull << 62;            // aggregate published
constexpr uint64_t kFlagP = 2ull << 62;            // inclusive prefix published
constexpr uint64_t kValMask = (1ull << 62) - 1;
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr uint32_t kAnchorTiles = 64;                // tiles that always resolve their prefix
constexpr uint32_t kStagedRecs = 16;                 // records a tile may stage for later placement
constexpr size_t kWsHeader = 256;
constexpr size_t kLdsLimit = 60 * 1024;   // dynamic LDS per block (static use is < 1 KB)

struct EncodeArgs {
    const void* w;
    uint32_t groups;
    uint32_t gpr;
    FastDiv gpr_div;
    FastDiv gpb_div;
    const float* coef;        // per row fl32(kappa * fl32(1/s)), NaN for a bad row
    const int8_t* signs;      // nullptr: no rotation
    uint32_t cols;
    uint32_t core_bound;
    const uint16_t* tab;
    RankParams rp;
    uint32_t wpk;             // digit weights ub^3, ub^2, ub, 1 as bytes (fast path)
    uint32_t ka[2], kb[2];    // v_dot4 accumulators giving 2*(F index), 2*(G index base)
    uint16_t* core_idx;
    e8q_escape_t* esc;
    uint64_t esc_cap;
    unsigned long long* esc_count;
    int8_t* two_z;
    uint32_t* tile_counter;
    unsigned long long* tile_status;
    uint32_t* tile_total;     // escapes per tile
    uint32_t* staged;         // kStagedRecs records (5 words each) per tile
    uint32_t num_tiles;
    uint32_t* status;
};

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
    const uint32_t lo = __shfl_xor(uint32_t(v), m, 64);
    const uint32_t hi = __shfl_xor(uint32_t(v >> 32), m, 64);
    return (uint64_t(hi) << 32) | lo;
}

// Ballot mask (bit = physical lane) re-ordered by logical group position:
// logical = physical ^ 3 on lanes whose bit 2 is set, i.e. the bits of every
// odd nibble are reversed.
__device__ __forceinline__ uint64_t logical_lane_mask(uint64_t m) {
    constexpr uint64_t odd = 0xF0F0F0F0F0F0F0F0ull;
    const uint64_t keep = m & ~odd;
    const uint64_t x = m & odd;
    const uint64_t rev = ((x & 0x1010101010101010ull) << 3) | ((x & 0x2020202020202020ull) << 1) |
                         ((x & 0x4040404040404040ull) >> 1) | ((x & 0x8080808080808080ull) >> 3);
    return keep | rev;
}

// Packed bytes b0 (bits 0-7) and b1 (bits 16-23), each 2z + 64, as the int16
// pair (b0 - 64, b1 - 64).
__device__ __forceinline__ uint32_t unbias_i16x2(uint32_t v) {
    typedef short i16x2 __attribute__((ext_vector_type(2)));
    const i16x2 d = __builtin_bit_cast(i16x2, v) - i16x2{64, 64};
    return __builtin_bit_cast(uint32_t, d);
}

// Appends an escape to the tile's LDS list (slots past kStagedRecs are
// dropped: such a tile writes its records in pass 2).
__device__ __forceinline__ void list_escape(uint32_t& n, uint32_t* lg, uint4* lz, uint32_t g, const uint4& z) {
    const uint32_t slot = atomicAdd(&n, 1u);
    if (slot < kStagedRecs) {
        lg[slot] = g;
        lz[slot] = z;
    }
}

// Workspace reset and per-row coefficients.
__global__ void encode_init_kernel(uint32_t* counter, unsigned long long* tile_status, uint32_t num_tiles,
                                   unsigned long long* esc_count, uint32_t batch, const float* scale,
                                   float* coef, uint32_t rows_total, float kappa) {
    const uint32_t i0 = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t stride = gridDim.x * blockDim.x;
    if (i0 == 0) *counter = 0u;
    for (uint32_t i = i0; i < num_tiles; i += stride) tile_status[i] = 0ull;
    for (uint32_t i = i0; i < batch; i += stride) esc_count[i] = 0ull;
    for (uint32_t i = i0; i < rows_total; i += stride) {
        bool bad;
        const float c = row_coef(scale[i], kappa, bad);
        coef[i] = bad ? __uint_as_float(0x7FC00000u) : c;
    }
}

template <typename WT, int HB, bool LDS_TAB, bool FAST>
__global__ __launch_bounds__(kBlock, 6) void encode_kernel(EncodeArgs a) {
    extern __shared__ uint32_t s_dyn[];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_cnt[kItems * kWaves];
    __shared__ unsigned long long s_ball[kItems][kWaves];
    __shared__ unsigned long long s_excl;
    __shared__ uint32_t s_staged;
    // the tile's first kStagedRecs escapes as pass 1 finds them (any order):
    // group index and 2z as four words of int16 pairs
    __shared__ uint32_t s_nlist;
    __shared__ uint32_t s_listed;
    __shared__ uint32_t s_lg[kStagedRecs];
    __shared__ uint4 s_lz[kStagedRecs];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wv = tid >> 6;

    // LDS: [sign masks: cols/2 words][wide-block buffer: 8*kBlock floats][rank table]
    const uint32_t smask_words = HB > 0 ? a.cols / 2u : 0u;
    const uint32_t wide_words = HB > 128 ? 8u * kBlock : 0u;
    uint32_t* s_smask = s_dyn;
    float* s_wide = reinterpret_cast<float*>(s_dyn + smask_words);
    const uint16_t* tab = a.tab;
    if constexpr (HB > 0) {
        for (uint32_t i = tid; i < smask_words; i += kBlock) {
            const uint32_t s0 = uint32_t(uint8_t(a.signs[2 * i])) >> 7;
            const uint32_t s1 = uint32_t(uint8_t(a.signs[2 * i + 1])) >> 7;
            s_smask[i] = (s0 << 15) | (s1 << 31);
        }
    }
    if constexpr (LDS_TAB) {
        // 16-byte copies (both ends are 16-byte aligned), then the tail
        uint16_t* t16 = reinterpret_cast<uint16_t*>(s_dyn + smask_words + wide_words);
        const uint32_t n16 = a.rp.entries / 8u;
        for (uint32_t i = tid; i < n16; i += kBlock)
            reinterpret_cast<uint4*>(t16)[i] = reinterpret_cast<const uint4*>(a.tab)[i];
        for (uint32_t i = 8u * n16 + tid; i < a.rp.entries; i += kBlock) t16[i] = a.tab[i];
        tab = t16;
    }
    const LaneFwht lf = lane_fwht<(HB > 128 ? 128 : HB)>(lane);
    const uint32_t lane_off = (lane & ~15u) + lf.logical;
    const uint32_t lpos = wv * kWave + lane_off;
    uint32_t kav[2], kbv[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        asm volatile("v_mov_b32 %0, %1" : "=v"(kav[c]) : "s"(a.ka[c]));
        asm volatile("v_mov_b32 %0, %1" : "=v"(kbv[c]) : "s"(a.kb[c]));
    }
    const uint32_t glast = a.groups - 1u;

    for (;;) {
        __syncthreads();
        if (tid == 0) {
            s_tile = atomicAdd(a.tile_counter, 1u);
            s_nlist = 0u;
        }
        __syncthreads();
        const uint32_t tile = s_tile;
        if (tile >= a.num_tiles) break;
        const uint32_t tbase = tile * kTileGroups + lpos;

        uint32_t flags = 0;
        // Loads run one item ahead of the arithmetic; lanes past the end read
        // the last group instead (nothing is stored for them).
        uint32_t g1 = tbase;
        uint32_t r1 = fdiv(min(g1, glast), a.gpr_div);
        Raw w1 = load_raw<WT>(a.w, min(g1, glast));
        float c1 = a.coef[r1];
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const uint32_t g = g1;
            const bool live = g < a.groups;
            const uint64_t live_mask = __ballot(live);   // scalar: taken before the decoder's branches
            const uint32_t gl = min(g, glast);
            const uint32_t row = r1;
            const Raw raw = w1;
            const float craw = c1;
            if (j + 1 < kItems) {
                g1 = g + kBlock;
                const uint32_t gn = min(g1, glast);
                r1 = fdiv(gn, a.gpr_div);
                w1 = load_raw<WT>(a.w, gn);
                c1 = a.coef[r1];
            }
            float v[8];
            const uint32_t vsign = rotate_group<WT, HB>(s_smask, s_wide, raw, gl - row * a.gpr, lf, lpos, tid, v);
            const float cl = __uint_as_float(__float_as_uint(craw) ^ vsign);
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = v[i] * cl;

            bool escaped = false;
            uint32_t cidx = 0xFFFFu;
            bool done = false;
            if constexpr (FAST) {
                uint32_t t0, t1;
                bool d8;
                if (fast_point(x, t0, t1, d8)) {
                    const uint32_t qa = __builtin_amdgcn_udot4(t0, t0, 0u, false);
                    const uint32_t sa4 = __builtin_amdgcn_sad_u8(t0, 0u, 0u);
                    const uint32_t qt = __builtin_amdgcn_udot4(t1, t1, qa, false);
                    const uint32_t st = __builtin_amdgcn_sad_u8(t1, 0u, sa4);
                    // sum (t + 64)^2 - 128 sum (t + 64) + 8 * 64^2 = ||2z||^2
                    const uint32_t norm = qt - (st << 7) + 32768u;
                    // lanes past the end hold the last group's point, which may be
                    // outside the core: only points inside it index the rank table
                    const bool outside = norm > a.core_bound;
                    escaped = live && outside;
                    if (escaped) {
                        // 2z + 64 bytes -> int16 pairs
                        const uint4 z = make_uint4(unbias_i16x2(__builtin_amdgcn_perm(0u, t0, 0x0C010C00u)),
                                                   unbias_i16x2(__builtin_amdgcn_perm(0u, t0, 0x0C030C02u)),
                                                   unbias_i16x2(__builtin_amdgcn_perm(0u, t1, 0x0C010C00u)),
                                                   unbias_i16x2(__builtin_amdgcn_perm(0u, t1, 0x0C030C02u)));
                        list_escape(s_nlist, s_lg, s_lz, g, z);
                    }
                    const uint32_t na = qa - (sa4 << 7) + 16384u;
                    const uint32_t fi = __builtin_amdgcn_udot4(t0, a.wpk, d8 ? kav[0] : kav[1], false) >> 1;
                    const uint32_t gb = __builtin_amdgcn_udot4(t1, a.wpk, d8 ? kbv[0] : kbv[1], false) >> 1;
                    const uint32_t state = (na >> 1) + ((sa4 >> 1) & 1u);
                    if (!outside) cidx = uint32_t(tab[fi]) + uint32_t(tab[__umul24(state, a.rp.nh) + gb]);
                    done = true;
                }
            }
            if (!done) {
                int t[8];
                const uint32_t inv = exact_point(x, __builtin_isnan(craw), t);
                if (live) flags |= inv;
                const bool outside = norm_u32(t) > a.core_bound;
                escaped = live && outside;
                if (escaped) {
                    uint4 z;
                    z.x = (uint32_t(t[0]) & 0xFFFFu) | (uint32_t(t[1]) << 16);
                    z.y = (uint32_t(t[2]) & 0xFFFFu) | (uint32_t(t[3]) << 16);
                    z.z = (uint32_t(t[4]) & 0xFFFFu) | (uint32_t(t[5]) << 16);
                    z.w = (uint32_t(t[6]) & 0xFFFFu) | (uint32_t(t[7]) << 16);
                    list_escape(s_nlist, s_lg, s_lz, g, z);
                }
                if (!outside) cidx = core_rank(t, tab, a.rp);
                if (a.two_z && live) {
                    uint32_t f8 = 0;
                    *reinterpret_cast<uint2*>(a.two_z + uint64_t(g) * 8) = pack_i8x8(t, f8);
                    flags |= f8;
                }
            }
            // cidx is 0xFFFF exactly for the points outside the core (a rank is
            // below 65535), so it is also the escape flag
            if (live) a.core_idx[g] = uint16_t(cidx);
            const uint64_t mask = __ballot(cidx == 0xFFFFu) & live_mask;
            if (lane == 0) {
                s_cnt[j * kWaves + wv] = uint32_t(__popcll(mask));
                s_ball[j][wv] = mask;
            }
        }
        flush_status(flags, a.status);
        __syncthreads();

        // First wave: exclusive scan of the (item, wave) counts in ascending
        // group order, then the decoupled look-back for the tile offset.
        if (wv == 0) {
            const uint32_t c = s_cnt[lane];
            uint32_t incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off, 64);
                if (lane >= uint32_t(off)) incl += o;
            }
            s_cnt[lane] = incl - c;
            const unsigned long long total = __shfl(incl, 63, 64);
            // Escape counts per batch item: one atomic for a tile inside one
            // item, else one per (slice, item) pair. Slice `lane` holds groups
            // tile * kTileGroups + 64 * lane + [0, 64) in logical lane order.
            {
                const uint32_t t0g = tile * kTileGroups;
                const uint32_t bfirst = fdiv(t0g, a.gpb_div);
                if (bfirst == fdiv(min(t0g + (kTileGroups - 1u), glast), a.gpb_div)) {
                    if (lane == 0 && total != 0ull) atomicAdd(a.esc_count + bfirst, total);
                } else if (c != 0u) {
                    uint64_t lm = logical_lane_mask(s_ball[lane / kWaves][lane % kWaves]);
                    const uint32_t gs = t0g + 64u * lane;
                    while (lm) {
                        const uint32_t first = uint32_t(__ffsll((unsigned long long)lm) - 1);
                        const uint32_t b = fdiv(gs + first, a.gpb_div);
                        const uint32_t end = (b + 1u) * a.gpb_div.d - gs;
                        const uint64_t sel = end >= 64u ? lm : (lm & ((1ull << end) - 1ull));
                        atomicAdd(a.esc_count + b, (unsigned long long)__popcll(sel));
                        lm &= ~sel;
                    }
                }
            }
            unsigned long long excl = 0;
            bool timeout = false;
            bool staged = false;
            if (lane == 0) a.tile_total[tile] = uint32_t(total);
            if (tile == 0) {
                if (lane == 0)
                    __hip_atomic_store(a.tile_status, kFlagP | total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else if (total <= kStagedRecs && tile % kAnchorTiles != 0u) {
                // Few records: publish the aggregate, stage the records and
                // skip the look-back and its wait.  Successors look back past
                // this tile; every kAnchorTiles-th tile resolves its prefix,
                // so a look-back never runs far.
                if (lane == 0)
                    __hip_atomic_store(a.tile_status + tile, kFlagA | total, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                staged = total != 0ull;
            } else {
                if (lane == 0)
                    __hip_atomic_store(a.tile_status + tile, kFlagA | total, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                int64_t jj = int64_t(tile) - 1;
                uint32_t spins = 0;
                for (;;) {
                    const int64_t idx = jj - int64_t(lane);
                    const unsigned long long v =
                        idx >= 0 ? __hip_atomic_load(a.tile_status + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : kFlagP;
                    const uint32_t flag = uint32_t(v >> 62);
                    const uint64_t pm = __ballot(flag == 2u);
                    const uint64_t xm = __ballot(flag == 0u);
                    const uint32_t first_p = pm ? uint32_t(__ffsll((unsigned long long)pm) - 1) : 64u;
                    const uint64_t win = first_p >= 63 ? ~0ull : ((2ull << first_p) - 1ull);
                    if (xm & win) {
                        if (++spins > kSpinLimit) {
                            timeout = true;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                        continue;
                    }
                    unsigned long long val = ((win >> lane) & 1ull) ? (v & kValMask) : 0ull;
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1) val += shfl_xor_u64(val, off);
                    excl += val;
                    if (first_p < 64) break;
                    jj -= 64;
                }
                if (lane == 0)
                    __hip_atomic_store(a.tile_status + tile, kFlagP | ((excl + total) & kValMask), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            // A tile with at most kStagedRecs escapes has them all in the list:
            // ranked by group, they go to the staging slot or to their final
            // slots here, and pass 2 has nothing to do.
            const bool listed = total <= kStagedRecs;
            if (listed && lane < uint32_t(total)) {
                const uint32_t gme = s_lg[lane];
                uint32_t rank = 0;
                for (uint32_t k = 0; k < uint32_t(total); ++k) rank += s_lg[k] < gme ? 1u : 0u;
                uint32_t* dst = nullptr;
                if (staged)
                    dst = a.staged + (uint64_t(tile) * kStagedRecs + rank) * 5u;
                else if (excl + rank < a.esc_cap)
                    dst = reinterpret_cast<uint32_t*>(a.esc + excl + rank);
                else
                    atomicOr(a.status, uint32_t(E8Q_STATUS_ESC_OVERFLOW));
                if (dst) {
                    const uint4 z = s_lz[lane];
                    dst[0] = gme - fdiv(gme, a.gpb_div) * a.gpb_div.d;
                    dst[1] = z.x;
                    dst[2] = z.y;
                    dst[3] = z.z;
                    dst[4] = z.w;
                }
            }
            if (lane == 0) {
                s_excl = excl;
                s_staged = staged ? 1u : 0u;
                s_listed = listed ? 1u : 0u;
                if (timeout) atomicOr(a.status, uint32_t(E8Q_STATUS_LOOKBACK_TIMEOUT));
            }
        }
        __syncthreads();

        // Pass 2: records of the slices that have escapes (recomputed on the
        // exact path; blocks wider than 512 columns need the whole block, so
        // the condition is block-uniform for them and wave-uniform otherwise).
        uint32_t oflags = 0;
        const unsigned long long excl = s_excl;
        const bool staged = s_staged != 0u;
        const int items2 = s_listed != 0u ? 0 : kItems;   // block-uniform
        for (int j = 0; j < items2; ++j) {
            const uint64_t mask = s_ball[j][wv];
            bool any;
            if constexpr (HB > 512) {
                uint64_t all = 0;
#pragma unroll
                for (int k = 0; k < kWaves; ++k) all |= s_ball[j][k];
                any = all != 0ull;
            } else {
                any = mask != 0ull;
            }
            if (!any) continue;
            const uint32_t g = tbase + uint32_t(j) * kBlock;
            const uint32_t gl = min(g, glast);
            const uint32_t row = fdiv(gl, a.gpr_div);
            float v[8];
            const uint32_t vsign = rotate_group<WT, HB>(s_smask, s_wide, load_raw<WT>(a.w, gl), gl - row * a.gpr,
                                                        lf, lpos, tid, v);
            const float craw = a.coef[row];
            const float cl = __uint_as_float(__float_as_uint(craw) ^ vsign);
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = v[i] * cl;
            if ((mask >> lane) & 1ull) {
                int t[8];
                exact_point(x, __builtin_isnan(craw), t);
                // records go in group order: count escapes at lower logical positions
                const uint64_t lmask = logical_lane_mask(mask);
                const uint32_t rank_in_wave = uint32_t(__popcll(lmask & ((1ull << lane_off) - 1ull)));
                const uint32_t local = s_cnt[j * kWaves + wv] + rank_in_wave;
                const unsigned long long pos = excl + local;
                uint32_t* dst = nullptr;
                if (staged)
                    dst = a.staged + (uint64_t(tile) * kStagedRecs + local) * 5u;   // local < kStagedRecs
                else if (pos < a.esc_cap)
                    dst = reinterpret_cast<uint32_t*>(a.esc + pos);
                else
                    oflags |= E8Q_STATUS_ESC_OVERFLOW;
                if (dst) {
                    dst[0] = g - fdiv(g, a.gpb_div) * a.gpb_div.d;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[1 + i] = (uint32_t(t[2 * i]) & 0xFFFFu) | (uint32_t(t[2 * i + 1]) << 16);
                }
            }
        }
        flush_status(oflags, a.status);
    }
}

// Placement of the staged records, after the encode kernel: one wave per
// kAnchorTiles tiles, the first of which is an anchor with its inclusive
// prefix resolved; a running scan of the per-tile counts, 64 tiles at a time,
// gives each tile's first slot.
__global__ __launch_bounds__(256) void encode_place_kernel(EncodeArgs a) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t first = (uint64_t(blockIdx.x) * 4u + (threadIdx.x >> 6)) * kAnchorTiles;
    if (first >= a.num_tiles) return;   // wave-uniform
    unsigned long long run = (a.tile_status[first] & kValMask) - a.tile_total[first];
    for (uint32_t c = 0; c < kAnchorTiles && first + c < a.num_tiles; c += 64u) {
        const uint64_t t = first + c + lane;
        const uint32_t tot = t < a.num_tiles ? a.tile_total[t] : 0u;
        uint32_t incl = tot;   // at most 64 * 4096
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t o = __shfl_up(incl, off, 64);
            if (lane >= uint32_t(off)) incl += o;
        }
        const unsigned long long base = run + (incl - tot);
        run += __shfl(incl, 63, 64);
        if (t == first || tot == 0u || tot > kStagedRecs) continue;
        // the staging area and the record list never overlap: four records'
        // loads are issued before their stores
        const uint32_t* __restrict__ src = a.staged + t * kStagedRecs * 5u;
        uint32_t* __restrict__ dst = reinterpret_cast<uint32_t*>(a.esc);
        uint32_t flags = 0;
        for (uint32_t r0 = 0; r0 < tot; r0 += 4u) {
            uint32_t v[4][5];
#pragma unroll
            for (uint32_t k = 0; k < 4u; ++k)
                if (r0 + k < tot) {
#pragma unroll
                    for (int i = 0; i < 5; ++i) v[k][i] = src[(r0 + k) * 5u + uint32_t(i)];
                }
#pragma unroll
            for (uint32_t k = 0; k < 4u; ++k) {
                if (r0 + k >= tot) break;
                const unsigned long long pos = base + r0 + k;
                if (pos < a.esc_cap) {
#pragma unroll
                    for (int i = 0; i < 5; ++i) dst[pos * 5u + uint64_t(i)] = v[k][i];
                } else {
                    flags |= E8Q_STATUS_ESC_OVERFLOW;
                }
            }
        }
        if (flags) atomicOr(a.status, flags);
    }
}

// ------------------------------------------------------------------ host

namespace {

uint32_t tiles_for(int64_t batch, int64_t rows, int64_t cols) {
    const uint64_t groups = uint64_t(batch) * uint64_t(rows) * uint64_t(cols / 8);
    return uint32_t((groups + kTileGroups - 1) / kTileGroups);
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

template <typename WT, bool LDS, bool FAST>
void launch_encode(int hb, const EncodeArgs& a, size_t lds, hipStream_t st) {
    switch (hb) {
        case 0: launch_tiles(encode_kernel<WT, 0, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 8: launch_tiles(encode_kernel<WT, 8, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 16: launch_tiles(encode_kernel<WT, 16, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 32: launch_tiles(encode_kernel<WT, 32, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 64: launch_tiles(encode_kernel<WT, 64, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 128: launch_tiles(encode_kernel<WT, 128, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 256: launch_tiles(encode_kernel<WT, 256, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 512: launch_tiles(encode_kernel<WT, 512, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 1024: launch_tiles(encode_kernel<WT, 1024, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 2048: launch_tiles(encode_kernel<WT, 2048, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        case 4096: launch_tiles(encode_kernel<WT, 4096, LDS, FAST>, a, a.num_tiles, kBlock, lds, st); break;
        default: break;
    }
}

}  // namespace

// Workspace: [counter][tile status words][row coefficients][per-tile escape
// counts][staged records, kStagedRecs per tile].
size_t encode_ws_bytes(int64_t batch, int64_t rows, int64_t cols) {
    const size_t tiles = tiles_for(batch, rows, cols);
    return kWsHeader + align256(sizeof(unsigned long long) * tiles) +
           align256(sizeof(float) * size_t(batch) * size_t(rows)) + align256(sizeof(uint32_t) * tiles) +
           align256(sizeof(e8q_escape_t) * kStagedRecs * tiles);
}

}  // namespace e8q

extern "C" size_t e8q_encode_workspace_size(int64_t batch, int64_t rows, int64_t cols) {
    if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 8) return 0;
    return e8q::encode_ws_bytes(batch, rows, cols);
}

namespace e8q {
namespace {

e8q_status_t encode_impl(const void* w, e8q_dtype_t w_dtype, int64_t batch, int64_t rows, int64_t cols,
                         const float* row_scale, const int8_t* signs, int32_t had_block, int32_t core_bound,
                         uint16_t* core_idx_out, e8q_escape_t* esc_out, int64_t esc_capacity,
                         int64_t* esc_count_out, int8_t* two_z_out, void* workspace, size_t workspace_bytes,
                         uint32_t* status_dev, void* stream) {
    e8q_status_t st = check_shape(w, w_dtype, batch, rows, cols, row_scale, status_dev);
    if (st != E8Q_OK) return st;
    if (!core_idx_out || !esc_count_out || !workspace) return E8Q_ERR_INVALID;
    if (esc_capacity < 0 || (esc_capacity > 0 && !esc_out)) return E8Q_ERR_INVALID;
    if (core_bound < 0 || core_bound > 40) return E8Q_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return E8Q_ERR_INVALID;
    if (workspace_bytes < e8q_encode_workspace_size(batch, rows, cols)) return E8Q_ERR_INVALID;
    int hb = 0;
    if (signs) {
        st = check_block(signs, had_block, cols);
        if (st != E8Q_OK) return st;
        hb = had_block;
    }
    const DevTable* tab = get_table(core_bound, st);
    if (!tab) return st;
    const RankParams& rp = tab->p;

    const uint32_t gpr = uint32_t(cols / 8);
    const uint32_t rows_total = uint32_t(batch * rows);
    EncodeArgs a;
    a.w = w;
    a.groups = uint32_t(uint64_t(batch) * uint64_t(rows) * gpr);
    a.gpr = gpr;
    a.gpr_div = make_fastdiv(gpr);
    a.gpb_div = make_fastdiv(uint32_t(uint64_t(rows) * gpr));
    a.signs = signs;
    a.cols = uint32_t(cols);
    a.core_bound = uint32_t(core_bound);
    a.tab = tab->dptr;
    a.rp = rp;
    const uint32_t ub = rp.ub;
    a.wpk = (ub * ub * ub) | ((ub * ub) << 8) | (ub << 16) | (1u << 24);
    const uint32_t sumw = ub * ub * ub + ub * ub + ub + 1u;
    for (int c = 0; c < 2; ++c) {
        const uint32_t bias = uint32_t(int32_t(rp.tm[c]) - 64) * sumw;   // mod 2^32
        a.ka[c] = bias + 2u * uint32_t(c) * rp.nh;
        a.kb[c] = bias + 2u * (2u * rp.nh + uint32_t(c) * rp.nstate * rp.nh);
    }
    a.core_idx = core_idx_out;
    a.esc = esc_out;
    a.esc_cap = uint64_t(esc_capacity);
    a.esc_count = reinterpret_cast<unsigned long long*>(esc_count_out);
    a.two_z = two_z_out;
    char* ws = static_cast<char*>(workspace);
    a.num_tiles = tiles_for(batch, rows, cols);
    a.tile_counter = reinterpret_cast<uint32_t*>(ws);
    a.tile_status = reinterpret_cast<unsigned long long*>(ws + kWsHeader);
    const size_t coef_off = kWsHeader + align256(sizeof(unsigned long long) * a.num_tiles);
    float* coef = reinterpret_cast<float*>(ws + coef_off);
    a.coef = coef;
    const size_t total_off = coef_off + align256(sizeof(float) * size_t(rows_total));
    a.tile_total = reinterpret_cast<uint32_t*>(ws + total_off);
    a.staged = reinterpret_cast<uint32_t*>(ws + total_off + align256(sizeof(uint32_t) * a.num_tiles));
    a.status = status_dev;

    const size_t smask_bytes = (hb > 0 ? size_t(cols / 2) * 4 : 0) + (hb > 128 ? size_t(8 * kBlock) * 4 : 0);
    const size_t tab_bytes = size_t(rp.entries) * sizeof(uint16_t);
    if (smask_bytes > kLdsLimit) return E8Q_ERR_UNSUPPORTED;   // rows too wide for the LDS sign masks

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint32_t init_items = a.num_tiles;
    if (uint32_t(batch) > init_items) init_items = uint32_t(batch);
    if (rows_total > init_items) init_items = rows_total;
    launch(encode_init_kernel, dim3(grid_for(init_items, 256, 4)), dim3(256), 0, s, a.tile_counter,
                       a.tile_status, a.num_tiles, a.esc_count, uint32_t(batch), row_scale, coef, rows_total,
                       kappa_for(hb));

    const bool lds_tab = smask_bytes + tab_bytes <= kLdsLimit;
    const size_t lds = smask_bytes + (lds_tab ? tab_bytes : 0);
    const bool fast = lds_tab && w_dtype == E8Q_BF16 && !two_z_out && ub <= 6;
    if (w_dtype == E8Q_BF16) {
        if (fast) launch_encode<uint16_t, true, true>(hb, a, lds, s);
        else if (lds_tab) launch_encode<uint16_t, true, false>(hb, a, lds, s);
        else launch_encode<uint16_t, false, false>(hb, a, lds, s);
    } else {
        if (lds_tab) launch_encode<float, true, false>(hb, a, lds, s);
        else launch_encode<float, false, false>(hb, a, lds, s);
    }
    const uint64_t segments = (uint64_t(a.num_tiles) + kAnchorTiles - 1) / kAnchorTiles;
    launch(encode_place_kernel, dim3(unsigned((segments + 3) / 4)), dim3(256), 0, s, a);
    return launch_status();
}

// Scratch of the allocation-free entry point: one array per device, part of
// the device code object (so it exists from load time on and is never
// allocated by a call), shared by every call on that device.  Marked used: no
// kernel names it (they get its address as an argument), and the device
// compiler would otherwise drop it.
constexpr size_t kScratchBytes = size_t(E8Q_ENCODE_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) __attribute__((used)) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device with that device current (the array's host-side name is not a
// device address).
void* scratch_address() {
    static std::mutex mu;
    static void* addr[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

}  // namespace
}  // namespace e8q

extern "C" e8q_status_t e8q_encode_core_escape(const void* w, e8q_dtype_t w_dtype, int64_t batch,
                                               int64_t rows, int64_t cols, const float* row_scale,
                                               const int8_t* signs, int32_t had_block,
                                               int32_t core_bound, uint16_t* core_idx_out,
                                               e8q_escape_t* esc_out, int64_t esc_capacity,
                                               int64_t* esc_count_out, int8_t* two_z_out,
                                               void* workspace, size_t workspace_bytes,
                                               uint32_t* status_dev, void* stream) {
    return e8q::encode_impl(w, w_dtype, batch, rows, cols, row_scale, signs, had_block, core_bound, core_idx_out,
                            esc_out, esc_capacity, esc_count_out, two_z_out, workspace, workspace_bytes, status_dev,
                            stream);
}

extern "C" e8q_status_t e8q_encode_core_escape_noalloc(const void* w, e8q_dtype_t w_dtype, int64_t batch,
                                                       int64_t rows, int64_t cols, const float* row_scale,
                                                       const int8_t* signs, int32_t had_block,
                                                       int32_t core_bound, uint16_t* core_idx_out,
                                                       e8q_escape_t* esc_out, int64_t esc_capacity,
                                                       int64_t* esc_count_out, int8_t* two_z_out,
                                                       uint32_t* status_dev, void* stream) {
    const size_t need = e8q_encode_workspace_size(batch, rows, cols);
    if (need == 0) return E8Q_ERR_INVALID;
    if (need > e8q::kScratchBytes) return E8Q_ERR_SCRATCH;   // checked before anything touches the device
    void* ws = e8q::scratch_address();
    if (!ws) return E8Q_ERR_DEVICE;
    return e8q::encode_impl(w, w_dtype, batch, rows, cols, row_scale, signs, had_block, core_bound, core_idx_out,
                            esc_out, esc_capacity, esc_count_out, two_z_out, ws, e8q::kScratchBytes, status_dev,
                            stream);
}
